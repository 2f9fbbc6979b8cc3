"""Lockstep parity driver shared by the GPU parity tests.

Every step the GPU denoises the oracle's current canvas with the oracle's KV
cache loaded (lockstep on the whole state, so one legitimate near-tie flip
cannot cascade); appends start from the same state.  Checked per step: logits
within the dtype's tolerance, predictions never [MASK], the commit kernel
bit-exact, commits per the margin rules in tests/parity.py; after the GPU's own
prefill and after every append: the new KV slots within the dtype's tolerance.

`max_steps` stops a canvas early: both sides then fill its remaining masked
positions with the oracle's predictions, so the append is still compared.
`paged` gives every request its cache as pages of one shared pool, drawn in
a shuffled order (so neighbouring tokens of a request sit in unrelated pages).
`sample` lists the requests the oracle follows; the GPU still runs the whole
batch (the launch shapes of the full workload), the other requests evolve on
the GPU alone and are checked by the properties that hold for any request:
the commit kernel applies the rule exactly to the GPU's own confidences, only
[MASK] positions change, and the counts it reports are right.
"""
import numpy as np
import torch

import synth
from oracle import sampler as osampler
from oracle.model import OracleModel, OracleWeights
from tests.parity import LOGIT_TOL, StepReport, compare_commit, compare_logits, router_exemptions


def _kv_close(gseq, ost, T, dtype, what, lo=0):
    """GPU cache (keys and values as [L, Hkv, cap, dh], gathered from pages when
    paged) against the oracle's per-layer K/V over slots [lo, T): relative RMS
    error per layer and kind (an intermediate tensor: one near-tie router or
    fp8-code flip moves a few elements by a quantisation step, which a max-abs
    bound would charge to the whole cache)."""
    g = [t.float().cpu().numpy() for t in gseq.read_kv()]
    worst = 0.0
    for l in range(g[0].shape[0]):
        for kind, ref in ((0, ost.k[l]), (1, ost.v[l])):
            o = ref[:, lo:T]
            d = np.sqrt(np.mean((g[kind][l, :, lo:T] - o) ** 2))
            s = np.sqrt(np.mean(o ** 2))
            worst = max(worst, d / s)
    assert worst <= LOGIT_TOL[dtype], f"{what}: KV relative RMS error {worst:.3g}"
    return worst


def _load_cache(gseq, ost):
    """Lockstep on the cache too: the GPU request gets the oracle's K/V of the
    cached slots [0, T) (bf16-exact values for bf16/fp8 models)."""
    T = ost.T
    k = np.stack([ost.k[l][:, :T] for l in range(len(ost.k))])
    v = np.stack([ost.v[l][:, :T] for l in range(len(ost.v))])
    gseq.write_kv(torch.from_numpy(k).to(gseq.kv.dtype).cuda(), torch.from_numpy(v).to(gseq.kv.dtype).cuda())



def lockstep(run, label, max_steps=None, sample=None, weights=None, paged=False):
    from masked_block_diffusion_amd import DLM, KVPool, Rule

    cfg = run.model
    C, n = run.canvas, run.n_requests
    sample = list(range(n)) if sample is None else list(sample)
    steps = run.n_steps if max_steps is None else min(run.n_steps, max_steps)
    print(f"[parity] run={label} dtype={cfg.dtype} ffn={cfg.ffn} L={cfg.n_layers} d={cfg.d_model} "
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
    ws = gm.workspace(max(n * C, max(len(p) for p in prefixes)), cap)
    for r in range(n):
        if r in ost:
            om.prefill(ost[r], prefixes[r].numpy())
        gm.dlm_prefill(gseqs[r], prefixes[r].cuda(), ws)
    torch.cuda.synchronize()
    for r in sample:
        assert gseqs[r].T == ost[r].T
        _kv_close(gseqs[r], ost[r], ost[r].T, cfg.dtype, f"prefill request {r}")

    rule = Rule.for_run(run)
    sched = osampler.topk_schedule(C, run.n_steps)
    conf = torch.empty(n * C, dtype=torch.float32, device="cuda")
    pred = torch.empty(n * C, dtype=torch.int32, device="cuda")
    logits = torch.empty(n * C * cfg.vocab, dtype=torch.float32, device="cuda")
    ncom = torch.empty(n, dtype=torch.int32, device="cuda")
    nmask = torch.empty(n, dtype=torch.int32, device="cuda")
    moe = cfg.ffn == "moe"
    rdbg = torch.empty(cfg.n_layers * n * C * max(cfg.top_k, 1), dtype=torch.int32, device="cuda") if moe else None
    rlog = torch.empty(cfg.n_layers * n * C * max(cfg.n_experts, 1), dtype=torch.float32,
                       device="cuda") if moe else None
    gm.dlm_debug_router(rdbg, rlog, cfg.n_layers * n * C)
    totals = StepReport()
    for ci in range(run.n_canvases):
        canv = {r: np.full(C, cfg.mask_id, dtype=np.int32) for r in sample}
        for s in gseqs:
            s.canvas.fill_(cfg.mask_id)
        last_pred = {}
        for step in range(steps):
            outs = {r: om.denoise(ost[r], canv[r], debug=True) for r in sample}
            new = {r: osampler.commit(canv[r], outs[r][0], outs[r][1], cfg.mask_id, run, step)[0] for r in sample}
            for r in sample:
                gseqs[r].canvas.copy_(torch.from_numpy(canv[r]))
                _load_cache(gseqs[r], ost[r])
            g_before = [s.canvas.cpu().numpy() for s in gseqs]
            gm.dlm_denoise_step(gseqs, conf, pred, ws, logits)
            gm.dlm_commit(gseqs, conf, pred, rule, step, ncom, nmask)
            torch.cuda.synchronize()
            lg = logits.view(n, C, cfg.vocab)
            g_pred = pred.view(n, C).cpu().numpy()
            g_conf = conf.view(n, C).cpu().numpy().astype(np.float64)
            g_after = [s.canvas.cpu().numpy() for s in gseqs]
            g_router = rdbg.view(cfg.n_layers, n, C, cfg.top_k).cpu().numpy() if moe else None
            g_rlog = rlog.view(cfg.n_layers, n, C, cfg.n_experts) if moe else None
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
                ex = router_exemptions(None if g_router is None else g_router[:, r],
                                       None if g_rlog is None else g_rlog[:, r].cpu().numpy().astype(np.float64),
                                       dbg.router_sets, dbg.router_gap, dbg.router_logits, rep)
                compare_logits(lg[r].cpu().numpy(), dbg.logits, cfg.mask_id, cfg.dtype, rep, ex)
                compare_commit(canv[r], g_after[r], new[r], conf_o, dbg.logits, cfg.mask_id, run.rule,
                               sched[step], run.threshold, run.rule == "threshold" and step == run.n_steps - 1,
                               rep, ex, rep.logit_err, run.edit_threshold)
                assert not rep.problems, f"canvas {ci} step {step} request {r}: {rep.problems}"
                totals.exempt_tokens += rep.exempt_tokens
                totals.exempt_ranks += rep.exempt_ranks
                totals.router_exempt_rows += rep.router_exempt_rows
                totals.logit_err = max(totals.logit_err, rep.logit_err / max(rep.logit_scale, 1e-30))
                totals.rank_margin = max(totals.rank_margin, rep.rank_margin)
                totals.router_margin = max(totals.router_margin, rep.router_margin)
                del dbg
            del outs
            canv = new
            if run.rule == "threshold" and not any(np.any(c == cfg.mask_id) for c in canv.values()):
                break
        if steps == run.n_steps:
            assert not any(np.any(c == cfg.mask_id) for c in canv.values()), "masked positions left after the schedule"
        for r in range(n):
            if r in canv:
                c = canv[r]
                c[c == cfg.mask_id] = last_pred[r][c == cfg.mask_id]       # stopped early: fill like the oracle
                gseqs[r].canvas.copy_(torch.from_numpy(c))
                _load_cache(gseqs[r], ost[r])
                om.append(ost[r], c)
            else:
                g = gseqs[r].canvas
                gp = pred.view(n, C)[r]
                gseqs[r].canvas.copy_(torch.where(g == cfg.mask_id, gp, g))
        gm.dlm_append_canvas(gseqs, ws)
        torch.cuda.synchronize()
        for r in sample:
            assert gseqs[r].T == ost[r].T
            _kv_close(gseqs[r], ost[r], ost[r].T, cfg.dtype, f"append canvas {ci} request {r}",
                      lo=ost[r].T - C)
    assert gm.dlm_check_device_status() == 0
    print(f"[parity] run={label} max rel logit err {totals.logit_err:.3g}; exempt tokens "
          f"{totals.exempt_tokens}, exempt rank positions {totals.exempt_ranks}, router-exempt rows "
          f"{totals.router_exempt_rows}, largest rank margin applied {totals.rank_margin:.3g}, largest "
          f"router margin applied {totals.router_margin:.3g}", flush=True)
    gm.close()
    return totals
