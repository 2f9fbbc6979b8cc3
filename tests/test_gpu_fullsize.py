"""Parity at the full sizes of the benchmarked workloads, in the launch
configuration bench.py times (same batch rows, widths, vocabulary, prefix and
canvas lengths, so every kernel runs its real grid and tile choice):

  * dense 16-layer d=2048 bf16 model, whole depth: prefill of the 1024-token
    prompt, the first denoising steps of the 256-token canvas, and the append;
  * the 26B-class MoE (d=2560, 128 experts top-8 x 768 + shared 2048, vocab
    262144) at full width but two of its 32 layers (the oracle cannot hold all
    26B weights in float64): prefill of the 4096-token prompt, the first
    denoising steps, the append -- in bf16, and in fp8 with the threshold rule;
  * the 32-request batch (prefixes of 512..4096 tokens, 8192 canvas rows per
    step, every request's cache in 64-token pages of one pool) at full width,
    two layers: the GPU runs the whole batch, the oracle
    follows two of the requests (requests never interact, so each can be
    computed alone); the others are checked by the commit properties.

Each step's checks are those of tests/lockstep.py.  The layers a reduced-depth
model runs are exactly the full model's first layers (same seeded tensors).
"""
from dataclasses import replace

import pytest

import synth
from tests.lockstep import lockstep

pytestmark = pytest.mark.gpu


def _two_layers(run):
    return replace(run, model=replace(run.model, n_layers=2), n_canvases=1)


def test_fullsize_dense():
    lockstep(synth.get_run("dense"), "dense (full size)", max_steps=3)


def test_fullsize_moe_two_layers():
    lockstep(_two_layers(synth.get_run("moe")), "moe (full width, 2 layers)", max_steps=2)


def test_fullsize_moe_fp8_one_layer():
    """fp8 kernels at full width where one layer keeps a flipped activation
    code from reaching the other rows through attention."""
    run = replace(synth.get_run("moe-fp8"), n_canvases=1)
    run = replace(run, model=replace(run.model, n_layers=1))
    lockstep(run, "moe-fp8 (full width, 1 layer)", max_steps=2)


@pytest.mark.xfail(strict=False, reason=(
    "fp8 per-token activation codes decided on near-ties cascade: under relative noise of 1e-7 to 1e-5 "
    "(fp32 rounding and accumulation) the float64 oracle's own logits move by 0.29 to 0.45 against a "
    "tolerance of 0.33 at this size (tests/fp8_conditioning.py moe 2); the GPU measured 0.40"))
def test_fullsize_moe_fp8_two_layers():
    lockstep(_two_layers(synth.get_run("moe-fp8")), "moe-fp8 (full width, 2 layers)", max_steps=2)


def test_fullsize_batch32_two_layers():
    run = _two_layers(synth.get_run("moe-batch32"))
    lengths = synth.prefix_lengths(run)
    sample = [min(range(len(lengths)), key=lambda r: lengths[r]),      # shortest and longest prompts
              max(range(len(lengths)), key=lambda r: lengths[r])]
    lockstep(run, "moe-batch32 (full width, 2 layers, paged)", max_steps=2, sample=sample, paged=True)
