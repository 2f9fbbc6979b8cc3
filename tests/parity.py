"""Comparison rules between the HIP path and the oracle, step by step.

The rules (the workload definitions' parity bar):
  * logits: max |gpu - oracle| <= tol * max |oracle| over the vocabulary
    without [MASK]; tol = 1e-4 (fp32 models), 2e-2 (bf16), 6e-2 (fp8);
  * commits: positions and tokens bit-exact wherever the oracle's decision has
    a margin above 1e-3 in log-probability units -- the top-1/top-2 logit gap
    for the token, the rank-k/rank-(k+1) log-confidence gap for the top-k set,
    |log conf - log threshold| for the threshold rule;
  * a row whose router choice differs from the oracle's at a layer where the
    oracle's k-th/(k+1)-th router logit gap is below 1e-3 is exempt (the same
    kind of near-tie); any other routing difference is a failure.
Where a decision is exempt, only what is unique is compared: the number of
commits, and the decisive positions on either side of the boundary.

The 1e-3 margin is a floor.  The logits themselves may differ by up to the
dtype's tolerance, and a measured logit difference e moves any top-1/top-2 gap
by at most 2e and any log-confidence (max logit minus log-sum-exp) by at most
2e, hence a rank gap by at most 4e and a threshold gap by at most 2e.  A
decision whose oracle margin is below that bound is not decidable at the
model's precision, so the margin used is max(1e-3, bound) with e measured on
the step; the bound actually applied is reported.  The commit kernel itself is
checked with no tolerance at all, against the oracle's rule applied to the
GPU's own confidences and predictions.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Set

import numpy as np

MARGIN = 1e-3
LOGIT_TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


@dataclass
class StepReport:
    logit_err: float = 0.0
    logit_scale: float = 0.0
    exempt_tokens: int = 0
    exempt_ranks: int = 0
    router_exempt_rows: int = 0
    router_flips_decisive: int = 0
    rank_margin: float = MARGIN
    router_margin: float = MARGIN
    problems: List[str] = field(default_factory=list)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """Per row: largest minus second largest logit (mask column already -inf)."""
    part = -np.partition(-logits, 1, axis=-1)[:, :2]
    return part[:, 0] - part[:, 1]


def router_exemptions(gpu_sets: Optional[np.ndarray], gpu_logits: Optional[np.ndarray],
                      oracle_sets: List[np.ndarray], oracle_gaps: List[np.ndarray],
                      oracle_logits: List[np.ndarray], rep: StepReport) -> Set[int]:
    """Rows exempt because of a router near-tie flip.  gpu_sets: [L, rows, k]
    (any order); gpu_logits: [L, rows, E]; oracle_sets[l]: [rows, k] sorted;
    oracle_gaps[l]: [rows] k-th minus (k+1)-th logit; oracle_logits[l]: [rows, E].
    A flip is exempt when the oracle gap is below max(1e-3, 2 e_l), e_l the
    layer's measured max router-logit difference (a gap above 2 e_l cannot
    close).  Exempt rows are left out of e_l, since a flip earlier in the
    forward legitimately changes a row's later router inputs."""
    rows: Set[int] = set()
    if gpu_sets is None or not oracle_sets:
        return rows
    for l, (os_, gap) in enumerate(zip(oracle_sets, oracle_gaps)):
        g = np.sort(gpu_sets[l], axis=-1)
        keep = np.array([r not in rows for r in range(len(gap))])
        e = float(np.max(np.abs(gpu_logits[l][keep] - oracle_logits[l][keep]))) if keep.any() else 0.0
        margin = max(MARGIN, 2.0 * e)
        rep.router_margin = max(rep.router_margin, margin)
        diff = np.any(g != os_, axis=-1)
        for r in np.nonzero(diff)[0]:
            if r in rows:
                continue
            if gap[r] < margin:
                rows.add(int(r))
            else:
                rep.router_flips_decisive += 1
                rep.problems.append(f"layer {l} row {r}: router set differs with oracle gap {gap[r]:.3g} "
                                    f"(margin {margin:.3g})")
    rep.router_exempt_rows = len(rows)
    return rows


def compare_logits(gpu: np.ndarray, oracle: np.ndarray, mask_id: int, dtype: str,
                   rep: StepReport, exempt_rows: Set[int] = frozenset()) -> None:
    keep = np.ones(oracle.shape[1], dtype=bool)
    keep[mask_id] = False
    rows = np.array([r for r in range(oracle.shape[0]) if r not in exempt_rows], dtype=np.int64)
    o = oracle[rows][:, keep]
    g = gpu[rows][:, keep]
    scale = float(np.max(np.abs(o))) if o.size else 0.0
    err = float(np.max(np.abs(g - o))) if o.size else 0.0
    rep.logit_err, rep.logit_scale = err, scale
    if err > LOGIT_TOL[dtype] * scale:
        rep.problems.append(f"logits: max|d| {err:.4g} > {LOGIT_TOL[dtype]} * {scale:.4g}")


def compare_commit(before: np.ndarray, gpu_after: np.ndarray, oracle_after: np.ndarray,
                   oracle_conf: np.ndarray, oracle_logits: np.ndarray, mask_id: int,
                   rule: str, k: int, threshold: float, forced: bool, rep: StepReport,
                   exempt_rows: Set[int] = frozenset(), logit_err: float = 0.0,
                   edit_threshold: float = 0.0) -> None:
    """One request's canvas before and after the commit, on both sides.
    logit_err: the step's measured max |gpu - oracle| logit difference.
    edit_threshold > 0: token editing is on, and the earlier tokens are
    compared like the commits (the edit decision is exempt where the oracle's
    confidence is within the margin of the threshold or its argmax is a
    near-tie)."""
    rank_m = max(MARGIN, 4.0 * logit_err)
    thr_m = max(MARGIN, 2.0 * logit_err)
    tok_m = max(MARGIN, 2.0 * logit_err)
    rep.rank_margin = max(rep.rank_margin, rank_m)
    masked = before == mask_id
    if not edit_threshold > 0.0:
        # positions that were not masked never change
        if np.any(gpu_after[~masked] != before[~masked]):
            rep.problems.append("commit changed a non-masked position")
    else:
        held = ~masked
        lc_e = np.log(np.maximum(oracle_conf, 1e-300))
        amb = held & ((np.abs(lc_e - np.log(edit_threshold)) <= thr_m) | (top2_margin(oracle_logits) <= tok_m))
        for r in exempt_rows:
            amb[r] = True
        g_ed = held & (gpu_after != before)
        o_ed = held & (oracle_after != before)
        if np.any((g_ed != o_ed) & ~amb):
            rep.problems.append(f"edit sets differ at decisive positions {np.nonzero((g_ed != o_ed) & ~amb)[0][:10].tolist()}")
        if np.any(g_ed & o_ed & ~amb & (gpu_after != oracle_after)):
            rep.problems.append("edited tokens differ")
        rep.exempt_tokens += int((amb & (g_ed | o_ed)).sum())
    g_set = masked & (gpu_after != mask_id)
    o_set = masked & (oracle_after != mask_id)
    lc = np.log(np.maximum(oracle_conf, 1e-300))
    idx = np.nonzero(masked)[0]
    order = sorted(idx.tolist(), key=lambda j: (-oracle_conf[j], j))
    ambiguous = np.zeros_like(masked)
    if forced:
        pass                                    # every masked position commits
    elif rule == "topk":
        if len(order) > k > 0:
            hi, lo = lc[order[k - 1]], lc[order[k]]
            if hi - lo <= rank_m:
                band = (lc >= lo - rank_m) & (lc <= hi + rank_m) & masked
                ambiguous |= band
                rep.exempt_ranks += int(band.sum())
        if int(g_set.sum()) != min(k, len(order)):
            rep.problems.append(f"top-k committed {int(g_set.sum())}, expected {min(k, len(order))}")
    else:
        near = masked & (np.abs(lc - np.log(threshold)) <= thr_m)
        ambiguous |= near
        if len(order) > 1 and not np.any(oracle_conf[idx] >= threshold):
            # the at-least-one rule picks the most confident position
            if lc[order[0]] - lc[order[1]] <= rank_m:
                band = masked & (lc >= lc[order[0]] - 2 * rank_m)
                ambiguous |= band
        rep.exempt_ranks += int(ambiguous.sum())
    for r in exempt_rows:
        ambiguous[r] = True
    bad = (g_set != o_set) & ~ambiguous
    if np.any(bad):
        rep.problems.append(f"commit sets differ at decisive positions {np.nonzero(bad)[0][:10].tolist()}")
    both = g_set & o_set
    tm = top2_margin(oracle_logits)
    decisive_tok = both & (tm > tok_m) & ~np.isin(np.arange(len(before)), list(exempt_rows))
    rep.exempt_tokens += int((both & (tm <= tok_m)).sum())
    wrong = decisive_tok & (gpu_after != oracle_after)
    if np.any(wrong):
        rep.problems.append(f"committed tokens differ at {np.nonzero(wrong)[0][:10].tolist()}")
