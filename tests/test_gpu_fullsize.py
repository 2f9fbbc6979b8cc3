"""Parity at the full sizes of the benchmarked workloads, in the launch
configuration bench.py times (same batch rows, widths, vocabulary, prefix and
canvas lengths, so every kernel runs its real grid and tile choice):

  * dense 16-layer d=2048 bf16 model, whole depth: prefill of the 1024-token
    prompt, the first denoising steps of the 256-token canvas, and the append;
  * the 26B-class MoE (d=2560, 128 experts top-8 x 768 + shared 2048, vocab
    262144) at full width but two of its 32 layers (all 32 run in
    tests/test_gpu_depth.py with a shorter prompt): prefill of the 4096-token
    prompt, the first denoising steps, the append -- in bf16, and in fp8 with
    the threshold rule (one and two layers), and with MXFP4 routed experts;
  * the 32-request batch (prefixes of 512..4096 tokens, 8192 canvas rows per
    step, every request's cache in 64-token pages of one pool) at full width,
    two layers: the GPU runs the whole batch, the oracle follows two of the
    requests (requests never interact, so each can be computed alone); the
    others are checked by the commit properties.

Each step's checks are those of tests/lockstep.py.  The layers a reduced-depth
model runs are exactly the full model's first layers (same seeded tensors).

Exempt-fraction caps: an implementation at fp32 accuracy (the oracle under an
independent fp32-level perturbation, judged with these rules on the CPU)
leaves 16% of the dense model's rank decisions and 12% of the two-layer MoE's
inside the bands, 2-5% of its tokens, 3% of the MoE rows router-exempt; the
caps allow for step-to-step spread.  fp8 at random init has confidences ~1e-3,
far below the 0.5 threshold, so each step's decision is the single most
confident position among near-equal ones: nearly all of them are inside the
bands (99% for the stand-in); fp8 runs report their fractions uncapped, and
their parity rests on the logits and on the kernel-level fp8 tests.
"""
from dataclasses import replace

import pytest

import synth
from tests.lockstep import lockstep

pytestmark = pytest.mark.gpu

BF16_CAPS = {"rank": 0.25, "token": 0.15, "router_rows": 0.10}
FP8_CAPS = {"router_rows": 0.15}


def _layers(run, n):
    return replace(run, model=replace(run.model, n_layers=n), n_canvases=1)


def test_fullsize_dense():
    lockstep(synth.get_run("dense"), "dense (full size)", max_steps=3, caps=BF16_CAPS)


def test_fullsize_moe_two_layers():
    lockstep(_layers(synth.get_run("moe"), 2), "moe (full width, 2 layers)", max_steps=2, caps=BF16_CAPS)


def test_fullsize_moe_mxfp4_two_layers():
    """The same two layers with the routed experts' weights in MXFP4: the
    prefill's 32768 assignments (several 64-row m-tiles per expert) and the
    canvas's 2048 through the MXFP4 grouped GEMM."""
    lockstep(_layers(synth.get_run("moe-mxfp4"), 2), "moe-mxfp4 (full width, 2 layers)", max_steps=2,
             caps=BF16_CAPS)


def test_fullsize_moe_mxfp6_two_layers():
    """The same two layers with MXFP6 (E2M3) routed experts."""
    lockstep(_layers(synth.get_run("moe-mxfp6"), 2), "moe-mxfp6 (full width, 2 layers)", max_steps=2,
             caps=BF16_CAPS)


def test_fullsize_moe_fp8_one_layer():
    lockstep(_layers(synth.get_run("moe-fp8"), 1), "moe-fp8 (full width, 1 layer)", max_steps=2, caps=FP8_CAPS)


def test_fullsize_moe_fp8_two_layers():
    """Two fp8 layers at full width: fp32-level noise flips activation E4M3
    codes in every canvas row and moves the oracle's own logits beyond
    6e-2 * max|logit| (measured on the CPU: 0.075); such steps are judged
    against twice the oracle's own move, measured at every step (see
    tests/parity.py, logit_bar)."""
    lockstep(_layers(synth.get_run("moe-fp8"), 2), "moe-fp8 (full width, 2 layers)", max_steps=2, caps=FP8_CAPS)


def test_fullsize_batch32_two_layers():
    run = _layers(synth.get_run("moe-batch32"), 2)
    lengths = synth.prefix_lengths(run)
    sample = [min(range(len(lengths)), key=lambda r: lengths[r]),      # shortest and longest prompts
              max(range(len(lengths)), key=lambda r: lengths[r])]
    lockstep(run, "moe-batch32 (full width, 2 layers, paged)", max_steps=2, sample=sample, paged=True,
             caps=BF16_CAPS)
