"""CPU checks of the parity rules themselves (tests/parity.py): the decision
bands measured on the oracle alone, what they accept and what they catch.
Mistakes are planted on the CPU, in copies of oracle outputs.

Stand-in for an implementation at fp32 accuracy: the oracle perturbed at fp32
level with an independent noise stream.  It must pass every rule with bands
measured from another perturbation (the GPU is held to the same bands), and
its exempt fractions are the ones the GPU runs are capped at."""
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle import sampler as osampler
from oracle.model import OracleModel, OracleWeights
from tests.parity import (MARGIN, Bands, StepReport, compare_commit, compare_logits, oracle_bands, perturbed, step_bands,
                          router_exemptions)


def _oracle(name, **model_changes):
    run = synth.get_run(name)
    if model_changes:
        run = replace(run, model=replace(run.model, **model_changes))
    cfg = run.model
    w = synth.make_weights(cfg, seed=run.seed)
    om = OracleModel(cfg, OracleWeights(cfg, w))
    st = om.new_seq(run.capacity())
    om.prefill(st, synth.make_inputs(run)[0].numpy())
    return run, cfg, om, st


def _step(om, st, canvas, seed=None):
    if seed is None:
        return om.denoise(st, canvas, debug=True)
    with perturbed(om, seed):
        return om.denoise(st, canvas, debug=True)


def test_perturbation_is_off_by_default_and_restored():
    run, cfg, om, st = _oracle("tiny")
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    a = _step(om, st, canvas)
    _step(om, st, canvas, seed=3)
    assert om.perturb is None
    b = _step(om, st, canvas)
    assert np.array_equal(a[2].logits, b[2].logits) and np.array_equal(a[0], b[0])


def test_bf16_model_moves_more_than_the_margin_under_fp32_noise():
    """fp32-sized relative noise (2^-20) on every contraction moves the bf16
    model's own log-confidences by more than 1e-3: such decisions cannot be
    bit-exact at this precision, whatever the implementation.  The move hardly
    depends on the noise size (1e-7 .. 1e-5 give the same order): it comes
    from bf16 storage roundings that any difference flips."""
    run, cfg, om, st = _oracle("dense-mini")
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    ex = _step(om, st, canvas)
    b = oracle_bands(cfg.mask_id, canvas == cfg.mask_id, ex, _step(om, st, canvas, seed=1))
    assert b.delta_lc > MARGIN
    assert 1e-4 < b.delta_logit_rel < 2e-2          # chaotic, yet well inside the bf16 logit tolerance
    assert b.rank == 4 * b.delta_lc and b.thr == 2 * b.delta_lc and b.tok == max(MARGIN, 2 * b.delta_gap)


def test_f32_model_bands_stay_at_the_floor():
    """The fp32 model stores nothing narrower than fp32: fp32-level noise moves
    its log-confidences far below 1e-3, so its bands are the 1e-3 floor."""
    run, cfg, om, st = _oracle("tiny")
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    b = oracle_bands(cfg.mask_id, canvas == cfg.mask_id, _step(om, st, canvas), _step(om, st, canvas, seed=1))
    assert b.delta_lc < 1e-5 and b.rank == MARGIN and b.tok == MARGIN


def _run_rules(name, steps, **model_changes):
    """Steps of a run where the 'implementation' is the oracle under an
    independent perturbation, judged with bands from another perturbation."""
    run, cfg, om, st = _oracle(name, **model_changes)
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    sched = osampler.topk_schedule(run.canvas, run.n_steps)
    tot = StepReport()
    for step in range(steps):
        exact = _step(om, st, canvas)
        bands = step_bands(om, st, canvas, exact, seed=11 + 10 * step)
        impl = _step(om, st, canvas, seed=5000 + step)
        rep = StepReport()
        ex = router_exemptions(None if not exact[2].router_sets else np.stack(impl[2].router_sets),
                               None if not exact[2].router_sets else np.stack(impl[2].router_logits),
                               exact[2], bands, cfg.dtype, rep)
        compare_logits(impl[2].logits, exact[2].logits, cfg.mask_id, cfg.dtype, rep, ex, bands)
        new, _ = osampler.commit(canvas, exact[0], exact[1], cfg.mask_id, run, step)
        got, _ = osampler.commit(canvas, impl[0], impl[1], cfg.mask_id, run, step)
        compare_commit(canvas, got, new, exact[0], exact[2].logits, cfg.mask_id, run.rule, sched[step],
                       run.threshold, run.rule == "threshold" and step == run.n_steps - 1, rep, bands, ex,
                       gpu_conf=impl[0])
        assert not rep.problems, f"{name} step {step}: {rep.problems}"
        tot.add(rep)
        canvas = new
    return tot


@pytest.mark.parametrize("name,steps", [("tiny", 8), ("dense-mini-ragged", 7), ("moe-mini", 6),
                                        ("dense-mini-fp8", 6), ("moe-mini-fp8", 6)])
def test_fp32_accurate_implementation_passes(name, steps):
    tot = _run_rules(name, steps)
    print(f"[rules] {name}: {tot.summary()}")
    # an independent perturbation moves about as far as the ones the bands came
    # from (a maximum over the few masked positions of a late step scatters)
    assert tot.gpu_lc_dev <= 4.0


def test_planted_logit_error_is_caught():
    run, cfg, om, st = _oracle("dense-mini-ragged")
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    dbg = _step(om, st, canvas)[2]
    bad = dbg.logits.copy()
    scale = np.max(np.abs(bad[:, np.arange(cfg.vocab) != cfg.mask_id]))
    bad[3, 7] += 0.03 * scale
    rep = StepReport()
    compare_logits(bad, dbg.logits, cfg.mask_id, "bf16", rep)
    assert rep.problems
    rep = StepReport()
    bad[3, cfg.mask_id] = 1e9            # the [MASK] column is not compared
    bad[3, 7] -= 0.03 * scale
    compare_logits(bad, dbg.logits, cfg.mask_id, "bf16", rep)
    assert not rep.problems


def test_planted_commit_mistakes_are_caught():
    run, cfg, om, st = _oracle("dense-mini-ragged")
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    conf, pred, dbg = exact = _step(om, st, canvas)
    bands = oracle_bands(cfg.mask_id, canvas == cfg.mask_id, exact, _step(om, st, canvas, seed=1))
    new, chosen = osampler.commit(canvas, conf, pred, cfg.mask_id, run, 0)
    k = len(chosen)
    order = np.argsort(-conf, kind="stable")
    lc = np.log(conf)
    # swap a decisive committed position (the most confident) for the least confident one
    assert lc[order[0]] - lc[order[-1]] > 2 * bands.rank
    bad = new.copy()
    bad[order[0]] = cfg.mask_id
    bad[order[-1]] = pred[order[-1]]
    rep = StepReport()
    compare_commit(canvas, bad, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep, bands)
    assert any("decisive" in p for p in rep.problems)
    # wrong token at a committed position with a clear top-1/top-2 gap
    tm = -np.partition(-dbg.logits, 1, axis=-1)[:, :2]
    gaps = tm[:, 0] - tm[:, 1]
    j = max(chosen.tolist(), key=lambda i: gaps[i])
    assert gaps[j] > bands.tok
    bad = new.copy()
    bad[j] = (pred[j] + 1) % (cfg.vocab - 1)
    rep = StepReport()
    compare_commit(canvas, bad, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep, bands)
    assert any("tokens differ" in p for p in rep.problems)
    # one commit too many
    bad = new.copy()
    extra = order[k]
    bad[extra] = pred[extra]
    rep = StepReport()
    compare_commit(canvas, bad, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep, bands)
    assert any("committed" in p for p in rep.problems)
    # a non-masked position changed
    before = new.copy()
    after = new.copy()
    after[chosen[0]] = (after[chosen[0]] + 1) % (cfg.vocab - 1)
    rep = StepReport()
    compare_commit(before, after, before, conf, dbg.logits, cfg.mask_id, "topk", 0, 0.5, False, rep, bands)
    assert any("non-masked" in p for p in rep.problems)
    # the band exempts only positions near the rank-k boundary: a swap across
    # the boundary inside the band passes, and is counted as exempt
    if lc[order[k - 1]] - lc[order[k]] <= bands.rank:
        ok = new.copy()
        ok[order[k - 1]] = cfg.mask_id
        ok[order[k]] = pred[order[k]]
        rep = StepReport()
        compare_commit(canvas, ok, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep, bands)
        assert not rep.problems and rep.exempt_ranks >= 2


def test_bands_do_not_grow_with_the_implementation_error():
    """The bands are a property of the oracle's step: a larger deviation of the
    implementation's confidences (the reported ratio) does not widen them, so
    a commit flipped outside them is caught."""
    run, cfg, om, st = _oracle("dense-mini-ragged")
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    conf, pred, dbg = exact = _step(om, st, canvas)
    bands = oracle_bands(cfg.mask_id, canvas == cfg.mask_id, exact, _step(om, st, canvas, seed=1))
    new, chosen = osampler.commit(canvas, conf, pred, cfg.mask_id, run, 0)
    k = len(chosen)
    lc = np.log(conf)
    order = np.argsort(-conf, kind="stable")
    # an implementation whose confidences are off by 10x the band
    wrong = np.exp(lc + 10 * bands.rank * np.where(np.arange(len(lc)) % 2 == 0, 1.0, -1.0))
    got, _ = osampler.commit(canvas, wrong, pred, cfg.mask_id, run, 0)
    rep = StepReport()
    compare_commit(canvas, got, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep, bands,
                   gpu_conf=wrong)
    assert rep.rank_band == bands.rank
    assert rep.gpu_lc_dev / bands.delta_lc > 5
    if not np.array_equal(got, new):
        assert any("decisive" in p for p in rep.problems) or lc[order[k - 1]] - lc[order[k]] <= bands.rank


def test_router_flip_rules():
    class D:       # an oracle StepDebug with one layer, two rows, four experts, k = 2
        router_sets = [np.array([[0, 1], [2, 3]])]
        router_gap = [np.array([5e-4, 0.5])]
        router_logits = [np.array([[1.0, 0.9, 0.1, 0.0], [0.0, 0.1, 1.0, 1.5]])]
    bands = Bands(delta_router=[0.0])
    # row 0 flips at a near-tie: exempt; row 1 flips at a wide gap: a failure
    g = np.array([[[0, 2], [2, 3]]])
    rep = StepReport()
    rows = router_exemptions(g, np.stack(D.router_logits), D, bands, "bf16", rep)
    assert rows == {0: 0} and not rep.problems
    g = np.array([[[0, 1], [1, 3]]])
    rep = StepReport()
    rows = router_exemptions(g, np.stack(D.router_logits), D, bands, "bf16", rep)
    assert rows == {} and rep.problems
    # a router band of 4 * 0.15 = 0.6 (from the oracle's own move, not the GPU's) exempts the 0.5-gap flip
    rep = StepReport()
    rows = router_exemptions(g, np.stack(D.router_logits), D, Bands(delta_router=[0.15]), "bf16", rep)
    assert rows == {1: 0} and not rep.problems
    # a choice a perturbed oracle run itself changed is exempt whatever its gap
    rep = StepReport()
    rows = router_exemptions(g, np.stack(D.router_logits), D, Bands(delta_router=[0.0], noisy_flips=[{1}]), "bf16",
                             rep)
    assert rows == {1: 0} and not rep.problems
    # router logits off by more than the tolerance at the flip layer are caught even when the flip is exempt
    glog = np.stack(D.router_logits).copy()
    glog[0, 1, 0] += 0.5
    rep = StepReport()
    router_exemptions(g, glog, D, Bands(delta_router=[0.15]), "bf16", rep)
    assert any("router logits differ" in p for p in rep.problems)


def test_logit_bar_is_the_tolerance_unless_the_oracle_itself_moves_beyond_it():
    from tests.parity import LOGIT_TOL, SAFETY, logit_bar
    assert logit_bar("bf16", None) == LOGIT_TOL["bf16"]
    assert logit_bar("bf16", Bands(delta_logit_rel=0.019)) == LOGIT_TOL["bf16"]
    assert logit_bar("fp8", Bands(delta_logit_rel=0.05)) == LOGIT_TOL["fp8"]
    assert logit_bar("fp8", Bands(delta_logit_rel=0.1)) == SAFETY * 0.1
    rep = StepReport()
    lg = np.zeros((2, 5)); lg[:, 4] = -np.inf
    ref = lg.copy(); ref[0, 0] = 1.0
    got = ref.copy(); got[1, 1] = 0.15                   # 0.15 of max|ref|: beyond 6e-2
    compare_logits(got, ref, 4, "fp8", rep, bands=Bands(delta_logit_rel=0.05))
    assert rep.problems
    rep = StepReport()
    compare_logits(got, ref, 4, "fp8", rep, bands=Bands(delta_logit_rel=0.1))   # the oracle moves 0.1 itself
    assert not rep.problems and rep.conditioned_steps == 1 and rep.logit_bar == SAFETY * 0.1


def test_fp8_noise_flips_codes_in_almost_every_row():
    """Why fp8 rows are not exempted by flipped E4M3 codes: fp32-level noise
    flips activation codes (the per-token quantisations over the whole canvas)
    in nearly every canvas row of the small two-layer fp8 MoE, so such an
    exemption would leave almost nothing to compare.  (At full width, d =
    2560 with two layers, every row flips thousands of codes and the oracle's
    own logits move beyond 6e-2 of their maximum: the conditioning bar of
    logit_bar, measured per step by the GPU tests.)"""
    import oracle.model as om_mod
    run, cfg, om, st = _oracle("moe-mini-fp8")
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    orig = om_mod.quant_per_token_e4m3
    logs = []
    try:
        for seed in (None, 1):
            log = []
            om_mod.quant_per_token_e4m3 = lambda a, log=log: (log.append(orig(a)) or log[-1])
            _step(om, st, canvas, seed)
            logs.append(log)
    finally:
        om_mod.quant_per_token_e4m3 = orig
    flipped = np.zeros(run.canvas, dtype=bool)
    for (q0, _), (q1, _) in zip(*logs):
        if q0.shape[0] == run.canvas and q0.shape == q1.shape:
            flipped |= np.any(q0 != q1, axis=1)
    assert flipped.mean() >= 0.9


def test_exempt_rows_may_displace_the_last_committed_ranks():
    """Top-k: a row whose routing flipped at a near-tie is exempt, and its GPU
    confidence may land anywhere, so it can push the oracle's last committed
    non-exempt row out of the GPU's top k: that row is inside the band (the
    rest of the ranking is still checked).  Without the exemption the same
    commit is a mistake."""
    C, mask = 6, 99
    before = np.full(C, mask, dtype=np.int32)
    conf = np.array([0.9, 0.8, 0.7, 0.6, 0.2, 0.1])
    logits = np.zeros((C, 100))
    logits[np.arange(C), np.arange(C)] = 5.0
    o_after = before.copy()
    o_after[:3] = [0, 1, 2]                      # the oracle commits its top 3
    g_after = before.copy()
    g_after[[0, 1, 5]] = [0, 1, 5]              # the GPU: row 5's confidence rose above row 2's
    for exempt, ok in (({5}, True), (set(), False)):
        rep = StepReport()
        compare_commit(before, g_after, o_after, conf, logits, mask, "topk", 3, 0.5, False, rep, Bands(),
                       exempt_rows=exempt)
        assert (not rep.problems) == ok, rep.problems
    # a second displaced row is still a mistake with one exempt row
    g_after = before.copy()
    g_after[[0, 4, 5]] = [0, 4, 5]
    rep = StepReport()
    compare_commit(before, g_after, o_after, conf, logits, mask, "topk", 3, 0.5, False, rep, Bands(),
                   exempt_rows={5})
    assert rep.problems
