"""CPU checks of the parity rules themselves (tests/parity.py) and of the reading
that widens the 1e-3 decision margin to what a measured logit difference can
move.  Mistakes are planted on the CPU, in copies of oracle outputs."""
import numpy as np

import synth
from oracle import sampler as osampler
from oracle.model import OracleModel, OracleWeights
from tests.parity import StepReport, compare_commit, compare_logits, router_exemptions


def _oracle_step(name="dense-mini-ragged"):
    run = synth.get_run(name)
    cfg = run.model
    w = synth.make_weights(cfg, seed=run.seed)
    om = OracleModel(cfg, OracleWeights(cfg, w))
    st = om.new_seq(run.capacity())
    om.prefill(st, synth.make_inputs(run)[0].numpy())
    canvas = np.full(run.canvas, cfg.mask_id, dtype=np.int32)
    conf, pred, dbg = om.denoise(st, canvas, debug=True)
    return run, cfg, om, canvas, conf, pred, dbg


def test_bf16_model_moves_more_than_the_margin_under_fp32_noise():
    """Relative noise of 2^-24 on every weight matrix (the size of fp32
    accumulation differences) moves the bf16 model's own log-confidences by
    more than 1e-3: such decisions cannot be bit-exact at this precision."""
    run, cfg, om, canvas, conf, _, dbg = _oracle_step("dense-mini")
    w = synth.make_weights(cfg, seed=run.seed)
    om2 = OracleModel(cfg, OracleWeights(cfg, w))
    rng = np.random.default_rng(1)
    for k, v in om2.W.w.items():
        if v.ndim >= 2 and k != "embed":
            om2.W.w[k] = v * (1 + rng.uniform(-2 ** -24, 2 ** -24, v.shape))
    st2 = om2.new_seq(run.capacity())
    om2.prefill(st2, synth.make_inputs(run)[0].numpy())
    conf2, _, dbg2 = om2.denoise(st2, canvas, debug=True)
    assert np.max(np.abs(np.log(conf) - np.log(conf2))) > 1e-3
    keep = np.arange(cfg.vocab) != cfg.mask_id
    rel = np.max(np.abs(dbg.logits[:, keep] - dbg2.logits[:, keep])) / np.max(np.abs(dbg.logits[:, keep]))
    assert 1e-4 < rel < 2e-2          # chaotic, yet well inside the bf16 logit tolerance


def test_identical_outputs_pass():
    run, cfg, _, canvas, conf, pred, dbg = _oracle_step()
    new, _ = osampler.commit(canvas, conf, pred, cfg.mask_id, run, 0)
    rep = StepReport()
    compare_logits(dbg.logits.copy(), dbg.logits, cfg.mask_id, cfg.dtype, rep)
    k = osampler.topk_schedule(run.canvas, run.n_steps)[0]
    compare_commit(canvas, new.copy(), new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep)
    assert not rep.problems


def test_planted_logit_error_is_caught():
    run, cfg, _, _, _, _, dbg = _oracle_step()
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
    run, cfg, _, canvas, conf, pred, dbg = _oracle_step()
    new, chosen = osampler.commit(canvas, conf, pred, cfg.mask_id, run, 0)
    k = len(chosen)
    order = np.argsort(-conf, kind="stable")
    lc = np.log(conf)
    # swap a decisive committed position (the most confident) for the least confident one
    bad = new.copy()
    bad[order[0]] = cfg.mask_id
    bad[order[-1]] = pred[order[-1]]
    rep = StepReport()
    compare_commit(canvas, bad, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep)
    assert any("decisive" in p for p in rep.problems)
    # wrong token at a committed position with a clear top-1/top-2 gap
    tm = -np.partition(-dbg.logits, 1, axis=-1)[:, :2]
    gaps = tm[:, 0] - tm[:, 1]
    j = max(chosen.tolist(), key=lambda i: gaps[i])
    bad = new.copy()
    bad[j] = (pred[j] + 1) % (cfg.vocab - 1)
    rep = StepReport()
    compare_commit(canvas, bad, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep)
    assert any("tokens differ" in p for p in rep.problems)
    # one commit too many
    bad = new.copy()
    extra = order[k]
    bad[extra] = pred[extra]
    rep = StepReport()
    compare_commit(canvas, bad, new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep)
    assert any("committed" in p for p in rep.problems)
    # a non-masked position changed
    before = new.copy()
    after = new.copy()
    after[chosen[0]] = (after[chosen[0]] + 1) % (cfg.vocab - 1)
    rep = StepReport()
    compare_commit(before, after, before, conf, dbg.logits, cfg.mask_id, "topk", 0, 0.5, False, rep)
    assert any("non-masked" in p for p in rep.problems)
    # the widened margin exempts only the band around the boundary
    rep = StepReport()
    e = 0.25 * (lc[order[k - 1]] - lc[order[k]]) if lc[order[k - 1]] > lc[order[k]] else 0.0
    compare_commit(canvas, new.copy(), new, conf, dbg.logits, cfg.mask_id, "topk", k, 0.5, False, rep,
                   logit_err=e)
    assert not rep.problems


def test_router_flip_rules():
    oracle_sets = [np.array([[0, 1], [2, 3]])]
    gaps = [np.array([5e-4, 0.5])]
    ologits = [np.zeros((2, 4))]
    # row 0 flips at a near-tie: exempt; row 1 flips at a wide gap: a failure
    g = np.array([[[0, 2], [2, 3]]])
    rep = StepReport()
    rows = router_exemptions(g, np.zeros((1, 2, 4)), oracle_sets, gaps, ologits, rep)
    assert rows == {0} and not rep.problems
    g = np.array([[[0, 1], [1, 3]]])
    rep = StepReport()
    rows = router_exemptions(g, np.zeros((1, 2, 4)), oracle_sets, gaps, ologits, rep)
    assert rows == set() and rep.problems
    # a measured router-logit difference of 0.3 widens the margin to 0.6: the 0.5-gap flip is exempt
    rep = StepReport()
    glog = np.zeros((1, 2, 4)); glog[0, 0, 0] = 0.3
    rows = router_exemptions(g, glog, oracle_sets, gaps, ologits, rep)
    assert rows == {1} and not rep.problems
