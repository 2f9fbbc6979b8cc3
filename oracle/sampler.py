"""Oracle commit rules and the generation loop.  TEST INFRASTRUCTURE ONLY.

  * Generation starts from an all-[MASK] block and repeatedly commits the
    positions the model is most confident about until nothing is masked
    ("Diffusion LLMs: what changes...", section 2, reverse process).  Commits go
    mask -> token only and are never reverted.
  * Several positions are committed per pass; tokens per forward pass is the
    figure of merit (same page, section 2, property 2).
  * A fixed step budget (up to 48 steps per 256-token canvas: same page,
    section 4.2 "Few steps"; b4rtaz.github.io "Diffusion LLMs are not a good fit
    for distributed inference", canvas paragraph).  The fixed-count rule splits
    C commits over S steps as evenly as possible, the larger counts first.
  * Confidence-threshold commits (same page, section 5, "Quality vs steps"):
    every masked position whose confidence reaches the threshold, at least the
    single most confident one, and every remaining position at the last step.
  * Ties in confidence rank go to the lower position.
  * Token editing (T2T; "Diffusion LLMs: what changes...", the LLaDA2.1 item:
    besides mask -> token commits the model may revise tokens it already
    wrote).  The pages give no rule; the plainest reading, used here: with an
    edit threshold tau > 0, every position that held a token before the step
    whose prediction differs from that token and whose confidence is at least
    tau is rewritten with the prediction, from the same forward pass as the
    step's commits.  Edits touch no [MASK] position and write no [MASK], so
    the masked count follows the commit rule exactly; tau = 0 turns editing
    off (mask -> token only, never reverted).

Pins: hand-built confidence vectors with known answers, and the invariants
(mask -> token only, counts per step equal the schedule, counts sum to C, no
[MASK] after the last step; with editing: the masked counts are those of the
commit rule alone, edits only rewrite earlier tokens with their prediction at
confidence >= tau) in tests/test_oracle_sampler.py.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def topk_schedule(canvas: int, n_steps: int) -> List[int]:
    """Commits per step: C // S everywhere, plus one on the first C % S steps."""
    base, extra = divmod(canvas, n_steps)
    return [base + (1 if s < extra else 0) for s in range(n_steps)]


def rank_masked(conf: np.ndarray, masked: np.ndarray) -> np.ndarray:
    """Masked positions ordered by confidence, highest first; equal confidence
    -> lower position first."""
    idx = np.nonzero(masked)[0]
    order = sorted(idx.tolist(), key=lambda j: (-float(conf[j]), j))
    return np.asarray(order, dtype=np.int64)


def commit_topk(canvas: np.ndarray, conf: np.ndarray, pred: np.ndarray, mask_id: int,
                k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Commit the k most confident masked positions (all of them if fewer are
    masked).  Returns (new canvas, committed positions)."""
    masked = canvas == mask_id
    chosen = rank_masked(conf, masked)[:k]
    out = canvas.copy()
    out[chosen] = pred[chosen]
    return out, chosen


def commit_threshold(canvas: np.ndarray, conf: np.ndarray, pred: np.ndarray, mask_id: int,
                     threshold: float, step: int, n_steps: int) -> Tuple[np.ndarray, np.ndarray]:
    """Commit every masked position with conf >= threshold; if there is none,
    the single most confident masked position; at the last step (index
    n_steps - 1) every masked position."""
    masked = canvas == mask_id
    order = rank_masked(conf, masked)
    if step >= n_steps - 1:
        chosen = order
    else:
        chosen = np.asarray([j for j in order if conf[j] >= threshold], dtype=np.int64)
        if len(chosen) == 0:
            chosen = order[:1]
    out = canvas.copy()
    out[chosen] = pred[chosen]
    return out, np.sort(chosen)


def edit_tokens(before: np.ndarray, conf: np.ndarray, pred: np.ndarray, mask_id: int,
                tau: float) -> np.ndarray:
    """Positions edited at this step: held a token before it, the prediction
    differs from that token, confidence >= tau (tau > 0; none for tau = 0)."""
    if not tau > 0.0:
        return np.zeros(0, dtype=np.int64)
    held = before != mask_id
    return np.nonzero(held & (pred != before) & (conf >= tau))[0].astype(np.int64)


def commit(canvas, conf, pred, mask_id, run, step):
    """The step's commits, plus token edits when the run has an edit
    threshold.  Returns (new canvas, committed positions)."""
    if run.rule == "topk":
        k = topk_schedule(run.canvas, run.n_steps)[step]
        out, chosen = commit_topk(canvas, conf, pred, mask_id, k)
    elif run.rule == "threshold":
        out, chosen = commit_threshold(canvas, conf, pred, mask_id, run.threshold, step, run.n_steps)
    else:
        raise ValueError(run.rule)
    edited = edit_tokens(canvas, conf, pred, mask_id, getattr(run, "edit_threshold", 0.0))
    if len(edited):
        out = out.copy()
        out[edited] = pred[edited]
    return out, chosen


def generate(model, run, prefix_ids, capacity=None, on_step=None, with_state=False):
    """Prefill the prefix, then for each canvas: start all-[MASK], denoise and
    commit until the schedule ends (or, for the threshold rule, until nothing is
    masked), then append the canvas to the KV cache.

    Returns (list of finished canvases, list of per-canvas step counts, state).
    `on_step(canvas_index, step, canvas_before, conf, pred, canvas_after)` sees
    every step; with `with_state` it also receives the request's state (its
    cache holds the prefix and the appended canvases up to T) and the step's
    debug record (logits, routing): on_step(..., canvas_after, state, dbg).
    """
    mask_id = model.cfg.mask_id
    st = model.new_seq(capacity or (len(prefix_ids) + run.n_canvases * run.canvas))
    model.prefill(st, np.asarray(prefix_ids))
    outs, steps = [], []
    for ci in range(run.n_canvases):
        canvas = np.full(run.canvas, mask_id, dtype=np.int32)
        s = 0
        for s in range(run.n_steps):
            conf, pred, dbg = model.denoise(st, canvas, debug=with_state)
            new, _ = commit(canvas, conf, pred, mask_id, run, s)
            if on_step is not None:
                if with_state:
                    on_step(ci, s, canvas, conf, pred, new, st, dbg)
                else:
                    on_step(ci, s, canvas, conf, pred, new)
            canvas = new
            if not np.any(canvas == mask_id):
                break
        steps.append(s + 1)
        model.append(st, canvas)
        outs.append(canvas)
    return outs, steps, st
