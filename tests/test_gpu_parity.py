"""End-to-end parity of the HIP path against the oracle, in lockstep (see
tests/lockstep.py for what is compared at every step).

Runs: the tiny fp32 model at its full size, and reduced bf16/fp8, dense/MoE
(MoE also with MXFP4 / MXFP6 routed experts and with a 2100-token prompt, whose
prefill takes the compute-bound expert tiles; dense also at head sizes 64 and 32),
single- and multi-request variants whose vocabulary, canvas and prefix sizes
are not multiples of any kernel tile; three of them again with paged caches.  The full-size workloads are in
tests/test_gpu_fullsize.py.
"""
import pytest

import synth
from tests.lockstep import lockstep

pytestmark = pytest.mark.gpu

RUNS = ["tiny", "dense-mini", "dense-mini-ragged", "moe-mini", "dense-mini-fp8", "moe-mini-fp8",
        "moe-mini-batch", "tiny-t2t", "moe-mini-mxfp4", "moe-mini-mxfp4-batch", "moe-mini-mxfp6",
        "moe-mini-mxfp6-batch", "dense-mini-dh64", "dense-mini-dh32", "moe-mini-longprompt"]


@pytest.mark.parametrize("name", RUNS)
def test_lockstep_parity(name):
    lockstep(synth.get_run(name), name)


@pytest.mark.parametrize("name", ["tiny", "dense-mini-ragged", "moe-mini-batch"])
def test_lockstep_parity_paged(name):
    """The same runs with every request's cache in 64-token pages of one pool,
    taken in a shuffled order."""
    lockstep(synth.get_run(name), name + " (paged)", paged=True)
