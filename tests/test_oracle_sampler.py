"""Pins for the oracle's commit rules and generation loop: hand-built confidence
vectors with known answers, the invariants the pages fix, and the pages' printed
figures (tests/golden/pages_figures.json)."""
import json
import os
from dataclasses import replace

import numpy as np
import pytest

import synth
from oracle.model import OracleModel, OracleWeights
from oracle.sampler import (commit, commit_threshold, commit_topk, edit_tokens, generate, rank_masked,
                            topk_schedule)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))
M = 99


def test_schedules():
    assert topk_schedule(256, 12) == [22] * 4 + [21] * 8
    assert topk_schedule(32, 8) == [4] * 8
    assert topk_schedule(256, 16) == [16] * 16
    for c in (1, 7, 40, 256):
        for s in (1, 3, 7, 12, 48):
            sch = topk_schedule(c, s)
            assert sum(sch) == c and max(sch) - min(sch) <= 1 and sch == sorted(sch, reverse=True)


def test_rank_ties_to_lower_position():
    conf = np.array([0.1, 0.5, 0.5, 0.3, 0.5])
    masked = np.array([True, True, True, True, False])
    assert rank_masked(conf, masked).tolist() == [1, 2, 3, 0]


def test_commit_topk_hand_built():
    canvas = np.array([M, 7, M, M, M, M])
    conf = np.array([0.2, 0.99, 0.2, 0.6, 0.1, 0.6])
    pred = np.array([10, 11, 12, 13, 14, 15])
    out, chosen = commit_topk(canvas, conf, pred, M, 3)
    assert sorted(chosen.tolist()) == [0, 3, 5]       # 0.6, 0.6, then 0.2 tie -> position 0
    assert out.tolist() == [10, 7, M, 13, M, 15]
    # asking for more than remain commits what remains
    out2, chosen2 = commit_topk(out, conf, pred, M, 10)
    assert sorted(chosen2.tolist()) == [2, 4] and not np.any(out2 == M)


def test_commit_threshold_hand_built():
    canvas = np.array([M, M, M, M])
    pred = np.array([1, 2, 3, 4])
    conf = np.array([0.5, 0.49, 0.7, 0.1])
    out, ch = commit_threshold(canvas, conf, pred, M, 0.5, step=0, n_steps=48)
    assert ch.tolist() == [0, 2]                       # >= is inclusive
    conf2 = np.array([0.3, 0.4, 0.4, 0.1])
    out, ch = commit_threshold(canvas, conf2, pred, M, 0.5, step=3, n_steps=48)
    assert ch.tolist() == [1]                          # none above: top-1, tie -> lower position
    out, ch = commit_threshold(canvas, conf2, pred, M, 0.5, step=47, n_steps=48)
    assert ch.tolist() == [0, 1, 2, 3]                 # last step: forced fill


def _tiny_run(rule="topk", steps=8, canvas=16):
    cfg = synth.configs.ModelConfig(
        name="t", n_layers=2, d_model=32, n_q_heads=4, n_kv_heads=2, head_dim=8,
        vocab=50, mask_id=49, ffn="dense", d_ffn=24, dtype="f32")
    run = synth.configs.RunConfig("t", cfg, canvas=canvas, n_requests=1, prefix_len=(9, 9),
                                  n_canvases=2, rule=rule, n_steps=steps)
    return run, OracleModel(cfg, OracleWeights(cfg, synth.make_weights(cfg)))


@pytest.mark.parametrize("rule,steps", [("topk", 8), ("topk", 5), ("threshold", 6)])
def test_generation_invariants(rule, steps):
    run, model = _tiny_run(rule, steps)
    mask = model.cfg.mask_id
    log = []

    def on_step(ci, s, before, conf, pred, after):
        assert np.all(pred != mask)
        changed = before != after
        assert np.all(before[changed] == mask)            # mask -> token only
        assert np.all(after[~changed] == before[~changed])  # nothing else moves
        assert np.all(after[changed] == pred[changed])
        log.append((ci, s, int(changed.sum())))

    ids = synth.prefix_ids(run, 0, 9).numpy()
    outs, nsteps, st = generate(model, run, ids, on_step=on_step)
    for ci, canvas in enumerate(outs):
        assert not np.any(canvas == mask)                  # nothing masked at the end
        counts = [n for c, s, n in log if c == ci]
        assert sum(counts) == run.canvas
        if rule == "topk":
            assert counts == topk_schedule(run.canvas, run.n_steps)
        else:
            assert all(n >= 1 for n in counts) and len(counts) <= run.n_steps
    assert st.T == 9 + 2 * run.canvas


def test_pages_figures_pin_tokens_per_pass():
    a = GOLDEN["table_a_distributed_gemma"]["rows"]
    steps = GOLDEN["table_b_steps"]["denoising_steps"]
    c = GOLDEN["table_b_steps"]["canvas"]
    tpf = np.mean(topk_schedule(c, steps))                # tokens committed per forward pass
    for row in a:                                         # bytes per pass / bytes per token
        assert abs(row["mb_per_pass"] / row["mb_per_token"] - tpf) < 0.05
    pp = GOLDEN["positions_per_token"]
    assert round(pp["canvas"] / pp["tpf"]) == pp["positions_per_token_approx"]
    # about 12 steps on average gives roughly 21 tokens per pass
    assert topk_schedule(256, GOLDEN["steps_budget"]["avg_steps"]) == [22] * 4 + [21] * 8
    cp = GOLDEN["compute_per_token"]
    assert abs(cp["diffusion_gflop_per_token"] / cp["ar_gflop_per_token"] - cp["ratio"]) < 0.1


def test_edit_tokens_hand_built():
    """Token editing: only positions that held a token, only where the
    prediction differs, only at confidence >= tau (inclusive); tau = 0 is off."""
    before = np.array([5, M, 6, 7, 8, M])
    pred = np.array([9, 1, 6, 3, 4, 2])
    conf = np.array([0.9, 0.99, 0.95, 0.2, 0.8, 0.1])
    assert edit_tokens(before, conf, pred, M, 0.8).tolist() == [0, 4]   # 2: same token; 3: 0.2 < 0.8
    assert edit_tokens(before, conf, pred, M, 0.85).tolist() == [0]
    assert edit_tokens(before, conf, pred, M, 0.0).tolist() == []
    run = synth.configs.RunConfig("e", None, canvas=6, n_requests=1, prefix_len=(1, 1), n_canvases=1,
                                  rule="topk", n_steps=2, edit_threshold=0.8)
    out, chosen = commit(before, conf, pred, M, run, 0)
    # commits: the 3 most confident masked positions of 2 (both); edits: 0 and 4
    assert sorted(chosen.tolist()) == [1, 5]
    assert out.tolist() == [9, 1, 6, 7, 4, 2]


@pytest.mark.parametrize("rule,steps", [("topk", 8), ("threshold", 6)])
def test_editing_invariants(rule, steps):
    """With editing on, the masked counts per step are those of the commit rule
    alone (edits neither fill nor create [MASK]), every change to an earlier
    token is its prediction at confidence >= tau, and the schedule still ends
    with no [MASK]; tau above every confidence reduces to mask -> token only."""
    run, om = _tiny_run(rule, steps)
    tau = 0.021                                   # inside the tiny model's confidence spread
    run_e = replace(run, edit_threshold=tau)
    prefix = np.arange(9) % 40
    seen = {"edits": 0}

    def check(ci, s, before, conf, pred, after):
        held = before != run.model.mask_id
        changed = before != after
        # the commit rule alone decides every masked position
        ref, _ = commit(before, conf, pred, run.model.mask_id, run, s)
        assert np.array_equal(after[~held], ref[~held])
        assert not np.any(after == run.model.mask_id) or np.sum(after == run.model.mask_id) == np.sum(ref == run.model.mask_id)
        ed = changed & held
        assert np.all(after[ed] == pred[ed]) and np.all(conf[ed] >= tau)
        keep = held & (pred != before) & (conf < tau)
        assert np.all(after[keep] == before[keep])
        seen["edits"] += int(ed.sum())

    outs, _, _ = generate(om, run_e, prefix, on_step=check)
    assert all(not np.any(c == run.model.mask_id) for c in outs)
    assert seen["edits"] > 0, "the threshold should let some edits through"
    outs_hi, _, _ = generate(om, replace(run, edit_threshold=2.0), prefix)
    outs_off, _, _ = generate(om, run, prefix)
    assert all(np.array_equal(a, b) for a, b in zip(outs_hi, outs_off))
