"""Lockstep parity driver shared by the GPU parity tests.

Every step the GPU denoises the oracle's current canvas with the oracle's KV
cache loaded (lockstep on the whole state, so one legitimate near-tie flip
cannot cascade); appends start from the same state.  Checked per step: logits
within the dtype's tolerance, predictions never [MASK], the commit kernel
bit-exact, commits per the rules and bands of tests/parity.py (the bands come
from the oracle run exactly and perturbed at fp32 level from the same state).

Prefill and append are checked element by element twice: the new KV slots
(every layer, keys and values) within the dtype's tolerance of the largest
oracle value of that layer and kind, and through the logits -- the first step
of every canvas is also run on the GPU's own cache (its own prefill for the
first canvas, its own append for the next ones) and its logits compared with
the oracle's like any step's.  For MoE models the routing of the prefill and
append forwards is compared too (every token, every layer that feeds the
cache): a token re-routed at a router near-tie is left out of the KV check
above the layer of the flip; any other routing difference fails.  Their bands
are those of the first step of the canvas (prefill) and of its last step
(append): the same model and layers, measured on the canvas rows.

`max_steps` stops a canvas early: both sides then fill its remaining masked
positions with the oracle's predictions, so the append is still compared.
`paged` gives every request its cache as pages of one shared pool, drawn in
a shuffled order (so neighbouring tokens of a request sit in unrelated pages).
`sample` lists the requests the oracle follows; the GPU still runs the whole
batch (the launch shapes of the full workload), the other requests evolve on
the GPU alone and are checked by the properties that hold for any request:
the commit kernel applies the rule exactly to the GPU's own confidences, only
[MASK] positions change, and the counts it reports are right.
`caps` bounds the exempt fractions ({"rank", "token", "router_rows"}); the
fractions are printed either way.
"""
from dataclasses import replace

import numpy as np
import torch

import synth
from oracle import sampler as osampler
from oracle.model import OracleModel, OracleWeights, StepDebug
from tests.parity import LOGIT_TOL, StepReport, compare_commit, compare_logits, router_exemptions, step_bands
from tests.progress import progress


def kv_check(gseq, ost, lo, hi, dtype, what, skip=None):
    """GPU cache slots [lo, hi) of every layer against the oracle's: max |d|
    per layer and kind (keys, values) within LOGIT_TOL of the largest oracle
    value of that layer and kind.  `skip` maps a slot (relative to lo) to the
    layer where its token was re-routed at a router near-tie: its K/V are
    compared up to that layer (they are computed before the layer's experts)
    and not above.  Returns the worst ratio to the bound."""
    g = [t.float().cpu().numpy() for t in gseq.read_kv()]
    worst = 0.0
    skip = skip or {}
    for l in range(g[0].shape[0]):
        keep = np.array([t for t in range(hi - lo) if skip.get(t, l) >= l], dtype=np.int64)
        if keep.size == 0:
            continue
        for kind, ref in ((0, ost.k[l]), (1, ost.v[l])):
            o = ref[:, lo:hi][:, keep]
            d = float(np.max(np.abs(g[kind][l, :, lo:hi][:, keep] - o)))
            bound = LOGIT_TOL[dtype] * float(np.max(np.abs(o)))
            assert d <= bound, (f"{what}: layer {l} {'KV'[kind]} max|d| {d:.4g} > {LOGIT_TOL[dtype]} * "
                                f"max|ref| = {bound:.4g}")
            worst = max(worst, d / max(bound, 1e-30))
    return worst


def cache_routing_flips(gpu_sets, gpu_logits, odbg, bands, dtype, what):
    """Routing of a prefill or append forward (GPU [L, rows, k] / [L, rows, E]
    against the oracle's StepDebug of the same forward) over the layers whose
    experts feed the cache -- all but the last, which the library skips there.
    Returns {row: layer of its near-tie flip}; fails on any other difference."""
    L = len(odbg.router_sets) - 1
    if L <= 0:
        return {}
    sub = StepDebug(None, odbg.router_sets[:L], odbg.router_gap[:L], odbg.router_logits[:L])
    rep = StepReport()
    flips = router_exemptions(gpu_sets[:L], gpu_logits[:L], sub, replace(bands, noisy_flips=[]), dtype, rep)
    assert not rep.problems, f"{what}: {rep.problems[:5]}"
    return flips


def load_cache(gseq, ost):
    """Lockstep on the cache too: the GPU request gets the oracle's K/V of the
    cached slots [0, T) (bf16-exact values for bf16/fp8 models)."""
    T = ost.T
    k = np.stack([ost.k[l][:, :T] for l in range(len(ost.k))])
    v = np.stack([ost.v[l][:, :T] for l in range(len(ost.v))])
    gseq.write_kv(torch.from_numpy(k).to(gseq.kv.dtype).cuda(), torch.from_numpy(v).to(gseq.kv.dtype).cuda())


def lockstep(run, label, max_steps=None, sample=None, weights=None, paged=False, caps=None):
    from masked_block_diffusion_amd import DLM, KVPool, Rule

    cfg = run.model
    L = cfg.n_layers
    C, n = run.canvas, run.n_requests
    sample = list(range(n)) if sample is None else list(sample)
    steps = run.n_steps if max_steps is None else min(run.n_steps, max_steps)
    print(f"[parity] run={label} dtype={cfg.dtype} ffn={cfg.ffn} L={L} d={cfg.d_model} "
          f"V={cfg.vocab} C={C} requests={n} sampled={sample} steps/canvas={steps} paged={paged}", flush=True)
    w = synth.make_weights(cfg, seed=run.seed) if weights is None else weights
    om = OracleModel(cfg, OracleWeights(cfg, w))
    gm = DLM(cfg, {k: v.cuda() for k, v in w.items()}, canvas=C)
    del w
    prefixes = synth.make_inputs(run)
    cap = run.capacity()
    ost = {r: om.new_seq(cap) for r in sample}
    if paged:
        per = -(-cap // 64)
        pool = KVPool(gm, n * per + 3)
        rng = np.random.default_rng(7)
        gseqs = [gm.new_seq(cap, pool, order=lambda nf: int(rng.integers(nf))) for _ in range(n)]
    else:
        gseqs = [gm.new_seq(cap) for _ in range(n)]
    rows_cap = max(n * C, max(len(p) for p in prefixes))
    ws = gm.workspace(rows_cap, cap)
    moe = cfg.ffn == "moe"
    rdbg = torch.empty(L * rows_cap * max(cfg.top_k, 1), dtype=torch.int32, device="cuda") if moe else None
    rlog = torch.empty(L * rows_cap * max(cfg.n_experts, 1), dtype=torch.float32, device="cuda") if moe else None
    gm.dlm_debug_router(rdbg, rlog, L * rows_cap)

    def routing(rows):
        """The last forward's routing: ([L, rows, k], [L, rows, E])."""
        torch.cuda.synchronize()
        return (rdbg[:L * rows * cfg.top_k].view(L, rows, cfg.top_k).cpu().numpy(),
                rlog[:L * rows * cfg.n_experts].view(L, rows, cfg.n_experts).cpu().numpy().astype(np.float64))

    pre_dbg, pre_route = {}, {}
    for r in range(n):
        progress(f"[parity] {label}: prefill request {r} ({len(prefixes[r])} tokens)")
        if r in ost:
            pre_dbg[r] = StepDebug() if moe else None
            om.prefill(ost[r], prefixes[r].numpy(), pre_dbg[r])
        gm.dlm_prefill(gseqs[r], prefixes[r].cuda(), ws)
        if moe and r in ost:
            pre_route[r] = routing(len(prefixes[r]))
    torch.cuda.synchronize()
    for r in sample:
        assert gseqs[r].T == ost[r].T

    rule = Rule.for_run(run)
    sched = osampler.topk_schedule(C, run.n_steps)
    conf = torch.empty(n * C, dtype=torch.float32, device="cuda")
    pred = torch.empty(n * C, dtype=torch.int32, device="cuda")
    logits = torch.empty(n * C * cfg.vocab, dtype=torch.float32, device="cuda")
    ncom = torch.empty(n, dtype=torch.int32, device="cuda")
    nmask = torch.empty(n, dtype=torch.int32, device="cuda")
    totals = StepReport()
    own_err = 0.0
    kv_worst = 0.0
    cache_flips = 0

    def router_views(r):
        if not moe:
            return None, None
        sets, lgs = routing(n * C)
        return sets.reshape(L, n, C, -1)[:, r], lgs.reshape(L, n, C, -1)[:, r]

    for ci in range(run.n_canvases):
        canv = {r: np.full(C, cfg.mask_id, dtype=np.int32) for r in sample}
        for s in gseqs:
            s.canvas.fill_(cfg.mask_id)
        last_pred, bands = {}, {}
        for step in range(steps):
            progress(f"[parity] {label}: canvas {ci} step {step}")
            outs = {r: om.denoise(ost[r], canv[r], debug=True) for r in sample}
            for r in sample:
                bands[r] = step_bands(om, ost[r], canv[r], outs[r], seed=100000 * ci + 100 * step + 10 * r)
            new = {r: osampler.commit(canv[r], outs[r][0], outs[r][1], cfg.mask_id, run, step)[0] for r in sample}
            if ci == 0 and step == 0:
                # the GPU's own prefill, element by element (now that bands exist)
                for r in sample:
                    skip = {}
                    if moe:
                        skip = cache_routing_flips(*pre_route[r], pre_dbg[r], bands[r], cfg.dtype,
                                                   f"prefill routing, request {r}")
                    cache_flips += len(skip)
                    kv_worst = max(kv_worst, kv_check(gseqs[r], ost[r], 0, ost[r].T, cfg.dtype,
                                                      f"prefill request {r}", skip))
            for r in sample:
                gseqs[r].canvas.copy_(torch.from_numpy(canv[r]))
            if step == 0:
                # the first step on the GPU's own cache: its prefill (first
                # canvas) or its append (later canvases) reaches the logits
                gm.dlm_denoise_step(gseqs, conf, pred, ws, logits)
                torch.cuda.synchronize()
                for r in sample:
                    rep = StepReport()
                    gs, gl = router_views(r)
                    ex = router_exemptions(gs, gl, outs[r][2], bands[r], cfg.dtype, rep)
                    compare_logits(logits.view(n, C, cfg.vocab)[r].cpu().numpy(), outs[r][2].logits, cfg.mask_id,
                                   cfg.dtype, rep, ex, bands[r])
                    assert not rep.problems, f"canvas {ci} first step on the GPU's own cache, request {r}: {rep.problems}"
                    own_err = max(own_err, rep.logit_err / max(rep.logit_scale, 1e-30))
            for r in sample:
                load_cache(gseqs[r], ost[r])
            g_before = [s.canvas.cpu().numpy() for s in gseqs]
            gm.dlm_denoise_step(gseqs, conf, pred, ws, logits)
            gm.dlm_commit(gseqs, conf, pred, rule, step, ncom, nmask)
            torch.cuda.synchronize()
            lg = logits.view(n, C, cfg.vocab)
            g_pred = pred.view(n, C).cpu().numpy()
            g_conf = conf.view(n, C).cpu().numpy().astype(np.float64)
            g_after = [s.canvas.cpu().numpy() for s in gseqs]
            assert np.all(g_pred != cfg.mask_id), "prediction is [MASK]"
            for r in range(n):
                # properties of every request: the commit kernel is exactly the rule
                # applied to the GPU's own conf / pred, and only [MASK] positions change
                want, _ = osampler.commit(g_before[r], g_conf[r], g_pred[r], cfg.mask_id, run, step)
                assert np.array_equal(want, g_after[r]), f"commit kernel differs at step {step} request {r}"
                changed = g_before[r] != g_after[r]
                if not run.edit_threshold > 0:
                    assert np.all(g_before[r][changed] == cfg.mask_id), "a committed position changed"
                assert int(ncom[r]) == int(changed.sum())
                assert int(nmask[r]) == int((g_after[r] == cfg.mask_id).sum())
            for r in sample:
                rep = StepReport()
                conf_o, pred_o, dbg = outs[r]
                last_pred[r] = pred_o
                gs, gl = router_views(r)
                ex = router_exemptions(gs, gl, dbg, bands[r], cfg.dtype, rep)
                compare_logits(lg[r].cpu().numpy(), dbg.logits, cfg.mask_id, cfg.dtype, rep, ex, bands[r])
                compare_commit(canv[r], g_after[r], new[r], conf_o, dbg.logits, cfg.mask_id, run.rule,
                               sched[step], run.threshold, run.rule == "threshold" and step == run.n_steps - 1,
                               rep, bands[r], ex, run.edit_threshold, gpu_conf=g_conf[r])
                assert not rep.problems, f"canvas {ci} step {step} request {r}: {rep.problems}"
                totals.add(rep)
                del dbg
            del outs
            canv = new
            if run.rule == "threshold" and not any(np.any(c == cfg.mask_id) for c in canv.values()):
                break
        if steps == run.n_steps:
            assert not any(np.any(c == cfg.mask_id) for c in canv.values()), "masked positions left after the schedule"
        app_dbg = {}
        for r in range(n):
            if r in canv:
                c = canv[r]
                c[c == cfg.mask_id] = last_pred[r][c == cfg.mask_id]       # stopped early: fill like the oracle
                gseqs[r].canvas.copy_(torch.from_numpy(c))
                load_cache(gseqs[r], ost[r])
                app_dbg[r] = StepDebug() if moe else None
                om.append(ost[r], c, app_dbg[r])
            else:
                g = gseqs[r].canvas
                gp = pred.view(n, C)[r]
                gseqs[r].canvas.copy_(torch.where(g == cfg.mask_id, gp, g))
        gm.dlm_append_canvas(gseqs, ws)
        torch.cuda.synchronize()
        app_route = routing(n * C) if moe else None
        for r in sample:
            assert gseqs[r].T == ost[r].T
            skip = {}
            if moe:
                sets, lgs = app_route
                skip = cache_routing_flips(sets.reshape(L, n, C, -1)[:, r], lgs.reshape(L, n, C, -1)[:, r],
                                           app_dbg[r], bands[r], cfg.dtype, f"append routing, canvas {ci} request {r}")
            cache_flips += len(skip)
            kv_worst = max(kv_worst, kv_check(gseqs[r], ost[r], ost[r].T - C, ost[r].T, cfg.dtype,
                                              f"append canvas {ci} request {r}", skip))
    assert gm.dlm_check_device_status() == 0
    progress(f"[parity] run={label} {totals.summary()}; first step on the GPU's own cache: max rel logit err "
          f"{own_err:.3g}; KV max|d| / bound {kv_worst:.3g} ({cache_flips} cached tokens re-routed at near-ties)")
    frac = totals.fractions()
    for key, cap_ in (caps or {}).items():
        assert frac[key] <= cap_, f"{label}: exempt {key} fraction {frac[key]:.3f} above the cap {cap_}"
    gm.close()
    return totals
