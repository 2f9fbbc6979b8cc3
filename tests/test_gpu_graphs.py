"""The step loop as HIP graph replays (CanvasSteps): every replay must give
exactly what the direct calls give.  The kernels are deterministic (fixed
reduction orders, no float atomics), so the comparison is bit-exact.

Each graph is replayed several times, with the program's own direct calls and
device synchronisations between the replays, and every replay is checked:
a captured graph re-issues its launches as recorded, so a launch that behaves
differently on a second replay shows up here.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def _setup(name, paged=False):
    from masked_block_diffusion_amd import DLM, KVPool, Rule
    run = synth.get_run(name)
    cfg = run.model
    gm = DLM(cfg, {k: v.cuda() for k, v in synth.make_weights(cfg, seed=run.seed).items()}, canvas=run.canvas)
    cap = run.capacity()
    pool = KVPool(gm, run.n_requests * (-(-cap // 64))) if paged else None
    seqs = [gm.new_seq(cap, pool) for _ in range(run.n_requests)]
    prefixes = [p.cuda() for p in synth.make_inputs(run)]
    ws = gm.workspace(max(run.n_requests * run.canvas, max(len(p) for p in prefixes)), cap)
    rule = Rule.for_run(run)
    return run, gm, seqs, prefixes, ws, rule


def _prefill(gm, seqs, prefixes, ws):
    for s, p in zip(seqs, prefixes):
        s.raw.T = 0
        gm.dlm_prefill(s, p, ws)
        s.canvas.fill_(gm.cfg.mask_id)


@pytest.mark.parametrize("name,paged", [("dense-mini", False), ("moe-mini-batch", True), ("tiny", False),
                                        ("moe-mini-mxfp4-batch", True), ("moe-mini-mxfp6", False)])
def test_step_graph_replays_match_direct_calls(name, paged):
    from masked_block_diffusion_amd import CanvasSteps
    run, gm, seqs, prefixes, ws, rule = _setup(name, paged)
    n, C = run.n_requests, run.canvas
    conf = torch.empty(n * C, dtype=torch.float32, device="cuda")
    pred = torch.empty(n * C, dtype=torch.int32, device="cuda")
    ncom = torch.empty(n, dtype=torch.int32, device="cuda")
    nmask = torch.empty(n, dtype=torch.int32, device="cuda")

    _prefill(gm, seqs, prefixes, ws)
    direct = []
    for step in range(rule.n_steps):
        gm.dlm_denoise_step(seqs, conf, pred, ws)
        gm.dlm_commit(seqs, conf, pred, rule, step, ncom, nmask)
        direct.append((conf.clone(), pred.clone(), torch.stack([s.canvas.clone() for s in seqs]),
                       ncom.clone(), nmask.clone()))
    torch.cuda.synchronize()

    _prefill(gm, seqs, prefixes, ws)
    torch.cuda.synchronize()
    cg = CanvasSteps(gm, seqs, conf, pred, rule, ws, ncom, nmask)
    for rep in range(3):
        for s in seqs:
            s.canvas.fill_(gm.cfg.mask_id)
        for step in range(rule.n_steps):
            cg.replay(step)
            torch.cuda.synchronize()
            want = direct[step]
            got = (conf, pred, torch.stack([s.canvas for s in seqs]), ncom, nmask)
            for what, a, b in zip(("conf", "pred", "canvas", "n_committed", "n_masked"), got, want):
                assert torch.equal(a, b), f"replay {rep} step {step}: {what} differs"
        # direct calls between replays (a canvas of other tokens), then synchronise
        for s in seqs:
            s.canvas.random_(0, gm.cfg.mask_id)
        gm.dlm_denoise_step(seqs, conf, pred, ws)
        torch.cuda.synchronize()
    assert gm.dlm_check_device_status() == 0
    gm.close()


def test_generate_with_graphs_matches_direct():
    """Two canvases (the second starts at a larger T, so it gets its own
    graphs), twice over with the same graph cache, against direct calls."""
    from masked_block_diffusion_amd import generate
    run, gm, seqs, prefixes, ws, rule = _setup("dense-mini")
    for s in seqs:
        s.raw.T = 0
    ref, ref_steps = generate(gm, seqs, prefixes, rule, run.n_canvases, ws)
    cache = {}
    for rep in range(2):
        for s in seqs:
            s.raw.T = 0
        out, steps = generate(gm, seqs, prefixes, rule, run.n_canvases, ws, graphs=cache)
        torch.cuda.synchronize()
        assert steps == ref_steps
        for ci, (a, b) in enumerate(zip(out, ref)):
            assert torch.equal(a, b), f"pass {rep} canvas {ci} differs"
    assert sorted(k for k in cache if isinstance(k, int)) == list(range(run.n_canvases))
    gm.close()


def test_graph_cache_recaptures_for_new_requests():
    """A graph cache kept across calls and handed fresh requests (same T, other
    canvases and caches) or another rule must not replay the old buffers: the
    results equal direct calls on the new requests."""
    from masked_block_diffusion_amd import Rule, generate
    run, gm, seqs, prefixes, ws, rule = _setup("dense-mini")
    cache = {}
    for s in seqs:
        s.raw.T = 0
    generate(gm, seqs, prefixes, rule, 1, ws, graphs=cache)
    fresh = [gm.new_seq(run.capacity()) for _ in seqs]
    ref, _ = generate(gm, [gm.new_seq(run.capacity()) for _ in seqs], prefixes, rule, 1, ws)
    out, _ = generate(gm, fresh, prefixes, rule, 1, ws, graphs=cache)
    torch.cuda.synchronize()
    assert torch.equal(out[0], ref[0])
    other = Rule.topk(run.canvas, run.n_steps // 2)
    ref2, _ = generate(gm, [gm.new_seq(run.capacity()) for _ in seqs], prefixes, other, 1, ws)
    out2, _ = generate(gm, [gm.new_seq(run.capacity()) for _ in seqs], prefixes, other, 1, ws, graphs=cache)
    torch.cuda.synchronize()
    assert torch.equal(out2[0], ref2[0])
    assert gm.dlm_check_device_status() == 0
    gm.close()
