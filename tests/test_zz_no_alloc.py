"""dlm_denoise_step_noalloc (the entry point for callers that cannot allocate)
against dlm_denoise_step with a caller workspace: the same kernels on the same
inputs, so conf, pred and logits must agree bit for bit -- on two calls in a
row, the second with a smaller input (fewer requests), since every call on the
device shares the one static array and the second call finds the first one's
contents there.  A pass needing more than the static maximum is refused
before anything is enqueued."""
import pytest
import torch

import synth
from masked_block_diffusion_amd import abi

pytestmark = pytest.mark.gpu


def _setup(name):
    from masked_block_diffusion_amd import DLM
    run = synth.get_run(name)
    cfg = run.model
    gm = DLM(cfg, {k: v.cuda() for k, v in synth.make_weights(cfg, seed=run.seed).items()}, canvas=run.canvas)
    cap = run.capacity()
    prefixes = synth.make_inputs(run)
    seqs = [gm.new_seq(cap) for _ in prefixes]
    ws = gm.workspace(max(len(seqs) * run.canvas, max(len(p) for p in prefixes)), cap)
    for s, p in zip(seqs, prefixes):
        gm.dlm_prefill(s, p.cuda(), ws)
    gen = torch.Generator(device="cpu").manual_seed(5)
    for s in seqs:            # a canvas half committed, half [MASK]
        c = torch.randint(0, cfg.vocab - 1, (run.canvas,), generator=gen, dtype=torch.int32)
        c[::2] = cfg.mask_id
        s.canvas.copy_(c.cuda())
    return run, cfg, gm, seqs, ws


def _outputs(run, cfg, n):
    C = run.canvas
    return (torch.full((n * C,), -1.0, device="cuda"), torch.full((n * C,), -1, dtype=torch.int32, device="cuda"),
            torch.full((n * C * cfg.vocab,), -1.0, device="cuda"))


@pytest.mark.parametrize("name", ["moe-mini-batch", "dense-mini-ragged", "tiny", "moe-mini-mxfp4-batch"])
def test_noalloc_matches_workspace_entry_point(name):
    run, cfg, gm, seqs, ws = _setup(name)
    for call, group in enumerate((seqs, seqs[:1])):       # the second call is smaller
        n = len(group)
        ref = _outputs(run, cfg, n)
        got = _outputs(run, cfg, n)
        gm.dlm_denoise_step(group, ref[0], ref[1], ws, ref[2])
        gm.dlm_denoise_step_noalloc(group, got[0], got[1], got[2])
        torch.cuda.synchronize()
        for a, b, what in zip(ref, got, ("conf", "pred", "logits")):
            assert torch.equal(a, b), f"{name} call {call}: {what} differs"
        assert gm.dlm_check_device_status() == 0
    gm.close()


def test_noalloc_refuses_a_pass_beyond_the_static_maximum():
    run, cfg, gm, seqs, ws = _setup("dense-mini")
    C = run.canvas
    n = next(k for k in range(1, abi.DLM_MAX_SEQS + 1)
             if gm.workspace_bytes(k * C, seqs[0].T + C) > abi.DLM_STATIC_SCRATCH_BYTES)
    many = [seqs[0]] * n                                   # only the host checks run
    conf, pred, _ = _outputs(run, cfg, n)
    with pytest.raises(abi.DLMError) as e:
        gm.dlm_denoise_step_noalloc(many, conf, pred)
    assert e.value.status == abi.DLM_E_WORKSPACE
    torch.cuda.synchronize()
    assert bool((conf == -1.0).all()) and bool((pred == -1).all())
    gm.close()
