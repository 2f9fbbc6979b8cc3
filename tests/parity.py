"""Comparison rules between the HIP path and the oracle, step by step.

The bar (the workload definitions' parity rule):
  * logits: max |gpu - oracle| <= tol * max |oracle| over the vocabulary
    without [MASK]; tol = 1e-4 (fp32 models), 2e-2 (bf16), 6e-2 (fp8);
  * commits: positions and tokens bit-exact wherever the oracle's decision has
    a margin above 1e-3 in log-probability units -- the top-1/top-2 logit gap
    for the token, the rank-k/rank-(k+1) log-confidence gap for the top-k set,
    |log conf - log threshold| for the threshold rule;
  * a row whose router choice differs from the oracle's at a layer where the
    oracle's k-th/(k+1)-th router logit gap is a near-tie is exempt (the same
    kind of near-tie); any other routing difference is a failure.

Decision bands.  1e-3 is a floor, not the band: a model stored in bf16 or fp8
cannot decide a 1e-3 margin reproducibly, because an fp32-sized difference
anywhere flips some storage rounding and the flips propagate.  The band of a
step is measured on the oracle alone, never on the GPU: the oracle runs the
step exactly and N_PERTURB more times from the same state with every
contraction result (GEMM outputs, router logits, attention outputs)
multiplied by (1 + EPS * N(0, 1)), EPS = 2^-20 -- the relative error an fp32
dot product of a few thousand terms carries -- each with its own noise
stream.  Over the perturbed runs: delta_lc is the largest move of a masked
position's log-confidence, delta_gap the largest move of a row's top-1 margin
(the exact argmax's logit minus the best other one), delta_router[l] the
largest move of a router logit at layer l over rows routed alike before l.
The GPU's fp32 arithmetic is another such perturbation; SAFETY (2, and 4 for
fp8, whose moves come in jumps of a flipped E4M3 code and scatter several-fold
between noise streams) covers its draw:
  rank band      2 * SAFETY * delta_lc   (both ends of a rank pair move)
  threshold band     SAFETY * delta_lc
  token band         SAFETY * delta_gap
  router band    2 * SAFETY * delta_router[l]
each at least 1e-3.  A router choice that a perturbed run itself changes is
undecidable at fp32 precision and exempt whatever its gap.  A decision inside
its band is exempt; only what is unique is then compared (the number of
commits, the decisive positions on either side).  Every run reports its
exempt fractions; the callers cap them.

Router-exempt rows keep a check: their router logits are compared with the
oracle's at every layer up to and including the layer of the flip (a flip
changes the row only after it); their final logits are not compared.  Their
confidence is unknown, so in a top-k step each of them may take the place of
one of the last committed rows (the last n_exempt non-exempt ranks above the
boundary are exempt), and under the threshold rule's at-least-one fallback
the oracle's top non-exempt row is exempt when any row is.

The commit kernel itself is checked with no tolerance at all, against the
oracle's rule applied to the GPU's own confidences and predictions.
"""
from __future__ import annotations

from contextlib import contextmanager
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Set

import numpy as np

MARGIN = 1e-3
LOGIT_TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
EPS = 2.0 ** -20
N_PERTURB = 3
SAFETY_OF = {"f32": 2.0, "bf16": 2.0, "fp8": 4.0}
SAFETY = SAFETY_OF["bf16"]


@contextmanager
def perturbed(om, seed: int):
    """Every contraction result of the oracle `om` carries relative noise
    EPS * N(0, 1) (seeded) inside the block."""
    rng = np.random.default_rng(seed)
    om.perturb = lambda y: y * (1.0 + EPS * rng.standard_normal(y.shape))
    try:
        yield om
    finally:
        om.perturb = None


def top2_margin(logits: np.ndarray) -> np.ndarray:
    """Per row: largest minus second largest logit (mask column already -inf)."""
    part = -np.partition(-logits, 1, axis=-1)[:, :2]
    return part[:, 0] - part[:, 1]


def pred_margin(logits: np.ndarray, pred: np.ndarray) -> np.ndarray:
    """Per row: logit of `pred` minus the largest other logit."""
    lg = logits.copy()
    r = np.arange(len(pred))
    top = lg[r, pred].copy()
    lg[r, pred] = -np.inf
    return top - lg.max(axis=-1)


@dataclass
class Bands:
    """An oracle step's sensitivity to fp32-level noise (see the module doc)."""
    delta_lc: float = 0.0
    delta_gap: float = 0.0
    delta_router: List[float] = field(default_factory=list)
    delta_logit_rel: float = 0.0
    safety: float = SAFETY
    noisy_flips: List[Set[int]] = field(default_factory=list)   # per layer: rows a perturbed run re-routed

    @property
    def rank(self) -> float:
        return max(MARGIN, 2 * self.safety * self.delta_lc)

    @property
    def thr(self) -> float:
        return max(MARGIN, self.safety * self.delta_lc)

    @property
    def tok(self) -> float:
        return max(MARGIN, self.safety * self.delta_gap)

    def router(self, layer: int) -> float:
        d = self.delta_router[layer] if layer < len(self.delta_router) else 0.0
        return max(MARGIN, 2 * self.safety * d)

    def noisy_flip(self, layer: int, row: int) -> bool:
        return layer < len(self.noisy_flips) and row in self.noisy_flips[layer]


def oracle_bands(mask_id: int, masked: np.ndarray, exact, noisy, dtype: str = "bf16") -> Bands:
    """Bands from the exact and the perturbed oracle outputs of one step:
    `exact` = (conf, pred, StepDebug) of OracleModel.denoise(debug=True),
    `noisy` = one or a list of the same from perturbed runs."""
    c0, p0, d0 = exact
    b = Bands(safety=SAFETY_OF[dtype])
    L = len(d0.router_sets)
    b.delta_router = [0.0] * L
    b.noisy_flips = [set() for _ in range(L)]
    lc0 = np.log(np.maximum(c0, 1e-300))
    keep = np.arange(d0.logits.shape[1]) != mask_id
    scale = max(np.max(np.abs(d0.logits[:, keep])), 1e-30)
    for c1, _, d1 in (noisy if isinstance(noisy, list) else [noisy]):
        same = np.ones(d0.logits.shape[0], dtype=bool)      # rows routed alike before the layer
        for l, (s0, s1, r0, r1) in enumerate(zip(d0.router_sets, d1.router_sets, d0.router_logits,
                                                  d1.router_logits)):
            if same.any():
                b.delta_router[l] = max(b.delta_router[l], float(np.max(np.abs(r1 - r0)[same])))
            flip = same & np.any(s0 != s1, axis=-1)
            b.noisy_flips[l].update(int(r) for r in np.nonzero(flip)[0])
            same &= ~flip
        # a row the perturbation re-routes at a router near-tie moves by a whole
        # expert's share: that is the router exemption's case, not fp32 noise
        lc1 = np.log(np.maximum(c1, 1e-300))
        if np.any(masked & same):
            b.delta_lc = max(b.delta_lc, float(np.max(np.abs(lc1 - lc0)[masked & same])))
        if np.any(same):
            b.delta_gap = max(b.delta_gap, float(np.max(
                np.abs(pred_margin(d1.logits, p0) - pred_margin(d0.logits, p0))[same])))
            b.delta_logit_rel = max(b.delta_logit_rel, float(np.max(
                np.abs(d1.logits[same][:, keep] - d0.logits[same][:, keep])) / scale))
    return b


def step_bands(om, st, canvas: np.ndarray, exact, seed: int, n: int = N_PERTURB) -> Bands:
    """Bands of the oracle step OracleModel.denoise(st, canvas) whose exact
    outputs are `exact`, from `n` perturbed runs (noise streams seed ..
    seed + n - 1).  The perturbed runs write the canvas's scratch K/V slots
    of `st` like any denoising pass; the cached slots are untouched."""
    noisy = []
    for i in range(n):
        with perturbed(om, seed + i):
            noisy.append(om.denoise(st, canvas, debug=True))
    return oracle_bands(om.cfg.mask_id, canvas == om.cfg.mask_id, exact, noisy, om.cfg.dtype)


@dataclass
class StepReport:
    logit_err: float = 0.0
    logit_scale: float = 0.0
    rank_decisions: int = 0
    exempt_ranks: int = 0
    token_decisions: int = 0
    exempt_tokens: int = 0
    router_rows: int = 0
    router_exempt_rows: int = 0
    router_flips_decisive: int = 0
    rank_band: float = MARGIN
    router_band: float = MARGIN
    gpu_lc_dev: float = 0.0            # max |log conf gpu - log conf oracle| over decided positions
    delta_lc: float = 0.0
    oracle_move: float = 0.0           # the oracle's own relative logit move under fp32-level noise
    conditioned_steps: int = 0         # steps judged against the conditioning bar (see logit_bar)
    logit_bar: float = 0.0
    problems: List[str] = field(default_factory=list)

    def add(self, o: "StepReport") -> None:
        for f in ("rank_decisions", "exempt_ranks", "token_decisions", "exempt_tokens", "router_rows",
                  "router_exempt_rows", "router_flips_decisive", "conditioned_steps"):
            setattr(self, f, getattr(self, f) + getattr(o, f))
        self.logit_err = max(self.logit_err, o.logit_err / max(o.logit_scale, 1e-30))
        self.rank_band = max(self.rank_band, o.rank_band)
        self.router_band = max(self.router_band, o.router_band)
        self.oracle_move = max(self.oracle_move, o.oracle_move)
        self.logit_bar = max(self.logit_bar, o.logit_bar)
        if o.delta_lc > 0:
            self.gpu_lc_dev = max(self.gpu_lc_dev, o.gpu_lc_dev / o.delta_lc)

    def fractions(self) -> Dict[str, float]:
        return {"rank": self.exempt_ranks / max(1, self.rank_decisions),
                "token": self.exempt_tokens / max(1, self.token_decisions),
                "router_rows": self.router_exempt_rows / max(1, self.router_rows)}

    def summary(self) -> str:
        f = self.fractions()
        cond = (f" (conditioning bar {self.logit_bar:.3g} on {self.conditioned_steps} step(s))"
                if self.conditioned_steps else "")
        return (f"max rel logit err {self.logit_err:.3g}, oracle's own move {self.oracle_move:.3g}{cond}; "
                f"exempt rank decisions {self.exempt_ranks}/"
                f"{self.rank_decisions} ({100 * f['rank']:.1f}%), exempt tokens {self.exempt_tokens}/"
                f"{self.token_decisions} ({100 * f['token']:.1f}%), router-exempt rows {self.router_exempt_rows}/"
                f"{self.router_rows}, largest rank band {self.rank_band:.3g}, largest router band "
                f"{self.router_band:.3g}, gpu log-conf deviation / oracle noise move {self.gpu_lc_dev:.2f}")


def router_exemptions(gpu_sets: Optional[np.ndarray], gpu_logits: Optional[np.ndarray], dbg, bands: Bands,
                      dtype: str, rep: StepReport) -> Dict[int, int]:
    """Rows exempt because of a router near-tie flip, mapped to the layer of
    their first flip.  gpu_sets: [L, rows, k] (any order), gpu_logits:
    [L, rows, E]; dbg: the exact oracle's StepDebug (router_sets sorted,
    router_gap = k-th minus (k+1)-th logit, router_logits) of the same rows.
    A flip at layer l is exempt when the oracle's gap is inside the layer's
    router band or a perturbed oracle run changed that row's choice at that
    layer too; every row's router logits are compared with the oracle's
    (LOGIT_TOL of the layer's largest) at every layer up to and including its
    first flip."""
    rows: Dict[int, int] = {}
    if gpu_sets is None or not dbg.router_sets:
        return rows
    n = len(dbg.router_gap[0])
    rep.router_rows += n
    first_flip = np.full(n, len(dbg.router_sets), dtype=np.int64)
    for l, (os_, gap) in enumerate(zip(dbg.router_sets, dbg.router_gap)):
        band = bands.router(l)
        rep.router_band = max(rep.router_band, band)
        live = first_flip >= l                  # rows not flipped before this layer
        ref = dbg.router_logits[l]
        scale = float(np.max(np.abs(ref[live]))) if live.any() else 0.0
        err = np.max(np.abs(gpu_logits[l] - ref), axis=-1)
        bad = live & (err > LOGIT_TOL[dtype] * scale)
        for r in np.nonzero(bad)[0][:5]:
            rep.problems.append(f"layer {l} row {r}: router logits differ by {err[r]:.3g} "
                                f"(tolerance {LOGIT_TOL[dtype] * scale:.3g})")
        diff = live & np.any(np.sort(gpu_sets[l], axis=-1) != os_, axis=-1)
        for r in np.nonzero(diff)[0]:
            first_flip[r] = l
            if gap[r] < band or bands.noisy_flip(l, int(r)):
                rows[int(r)] = l
            else:
                rep.router_flips_decisive += 1
                rep.problems.append(f"layer {l} row {r}: router set differs with oracle gap {gap[r]:.3g} "
                                    f"(band {band:.3g})")
    rep.router_exempt_rows += len(rows)
    return rows


def logit_bar(dtype: str, bands: Optional[Bands]) -> float:
    """Relative logit bar of a step: the dtype's tolerance, unless the oracle
    itself, perturbed at fp32 level, moves beyond it (a model too badly
    conditioned for that tolerance at fp32 precision -- the fp8 MoE past one
    layer at full width, where such noise flips E4M3 codes in every row); then
    SAFETY times the oracle's own move."""
    tol = LOGIT_TOL[dtype]
    if bands is not None and bands.delta_logit_rel > tol:
        return bands.safety * bands.delta_logit_rel
    return tol


def compare_logits(gpu: np.ndarray, oracle: np.ndarray, mask_id: int, dtype: str,
                   rep: StepReport, exempt_rows: Set[int] = frozenset(), bands: Optional[Bands] = None) -> None:
    keep = np.ones(oracle.shape[1], dtype=bool)
    keep[mask_id] = False
    rows = np.array([r for r in range(oracle.shape[0]) if r not in exempt_rows], dtype=np.int64)
    o = oracle[rows][:, keep]
    g = gpu[rows][:, keep]
    scale = float(np.max(np.abs(o))) if o.size else 0.0
    err = float(np.max(np.abs(g - o))) if o.size else 0.0
    rep.logit_err, rep.logit_scale = err, scale
    bar = logit_bar(dtype, bands)
    if bands is not None:
        rep.oracle_move = max(rep.oracle_move, bands.delta_logit_rel)
    if bar > LOGIT_TOL[dtype]:
        rep.conditioned_steps += 1
        rep.logit_bar = max(rep.logit_bar, bar)
    if err > bar * scale:
        rep.problems.append(f"logits: max|d| {err:.4g} > {bar:.3g} * {scale:.4g}"
                            + (" (conditioning bar)" if bar > LOGIT_TOL[dtype] else ""))


def compare_commit(before: np.ndarray, gpu_after: np.ndarray, oracle_after: np.ndarray,
                   oracle_conf: np.ndarray, oracle_logits: np.ndarray, mask_id: int,
                   rule: str, k: int, threshold: float, forced: bool, rep: StepReport, bands: Bands,
                   exempt_rows: Set[int] = frozenset(), edit_threshold: float = 0.0,
                   gpu_conf: Optional[np.ndarray] = None) -> None:
    """One request's canvas before and after the commit, on both sides.
    edit_threshold > 0: token editing is on, and the earlier tokens are
    compared like the commits (the edit decision is exempt where the oracle's
    confidence is within the threshold band of the edit threshold or its
    argmax is inside the token band).  gpu_conf: the GPU's confidences, for the
    reported deviation."""
    rank_m, thr_m, tok_m = bands.rank, bands.thr, bands.tok
    rep.rank_band = max(rep.rank_band, rank_m)
    rep.delta_lc = bands.delta_lc
    masked = before == mask_id
    ex = np.zeros(len(before), dtype=bool)
    ex[list(exempt_rows)] = True
    lc = np.log(np.maximum(oracle_conf, 1e-300))
    if gpu_conf is not None and np.any(masked & ~ex):
        d = np.abs(np.log(np.maximum(gpu_conf, 1e-300)) - lc)[masked & ~ex]
        rep.gpu_lc_dev = max(rep.gpu_lc_dev, float(d.max()))
    tm = pred_margin(oracle_logits, np.argmax(oracle_logits, axis=-1))
    if not edit_threshold > 0.0:
        # positions that were not masked never change
        if np.any(gpu_after[~masked] != before[~masked]):
            rep.problems.append("commit changed a non-masked position")
    else:
        held = ~masked
        amb = held & ((np.abs(lc - np.log(edit_threshold)) <= thr_m) | (tm <= tok_m)) | (held & ex)
        g_ed = held & (gpu_after != before)
        o_ed = held & (oracle_after != before)
        if np.any((g_ed != o_ed) & ~amb):
            rep.problems.append(f"edit sets differ at decisive positions {np.nonzero((g_ed != o_ed) & ~amb)[0][:10].tolist()}")
        if np.any(g_ed & o_ed & ~amb & (gpu_after != oracle_after)):
            rep.problems.append("edited tokens differ")
        rep.exempt_tokens += int((amb & (g_ed | o_ed)).sum())
        rep.token_decisions += int((g_ed | o_ed).sum())
    g_set = masked & (gpu_after != mask_id)
    o_set = masked & (oracle_after != mask_id)
    idx = np.nonzero(masked)[0]
    order = sorted(idx.tolist(), key=lambda j: (-oracle_conf[j], j))
    ambiguous = np.zeros_like(masked)
    decided = not forced and not (rule == "topk" and k >= len(order))
    if forced:
        pass                                    # every masked position commits
    elif rule == "topk":
        if len(order) > k > 0:
            hi, lo = lc[order[k - 1]], lc[order[k]]
            if hi - lo <= rank_m:
                ambiguous |= (lc >= lo - rank_m) & (lc <= hi + rank_m) & masked
            # an exempt row (re-routed at a near-tie) has no confidence to
            # compare, so it may hold any rank on the GPU: each one can push
            # one of the last committed rows out of the top k
            n_ex = int((ex & masked).sum())
            if n_ex:
                ne = [j for j in order if not ex[j]]
                ambiguous[ne[max(0, k - n_ex):k]] = True
        if int(g_set.sum()) != min(k, len(order)):
            rep.problems.append(f"top-k committed {int(g_set.sum())}, expected {min(k, len(order))}")
    else:
        ambiguous |= masked & (np.abs(lc - np.log(threshold)) <= thr_m)
        if len(order) > 1 and not np.any(oracle_conf[idx] >= threshold):
            # the at-least-one rule picks the most confident position: any
            # position within the rank band of it could take its place, and
            # so could an exempt row (on the GPU it may even pass the threshold)
            if lc[order[0]] - lc[order[1]] <= rank_m:
                ambiguous |= masked & (lc >= lc[order[0]] - rank_m)
            ne = [j for j in order if not ex[j]]
            if np.any(ex & masked) and ne:
                ambiguous[ne[0]] = True
    ambiguous |= ex & masked
    if decided:
        rep.rank_decisions += int(masked.sum())
        rep.exempt_ranks += int(ambiguous.sum())
    bad = (g_set != o_set) & ~ambiguous
    if np.any(bad):
        where = np.nonzero(bad)[0][:10].tolist()
        detail = ""
        if gpu_conf is not None:
            glc = np.log(np.maximum(gpu_conf, 1e-300))
            detail = (f" (oracle log-conf {[round(float(lc[j]), 5) for j in where]}, GPU's "
                      f"{[round(float(glc[j]), 5) for j in where]}; the oracle's {k}th / {k + 1}th "
                      f"{[round(float(lc[order[i]]), 5) for i in (k - 1, k) if 0 <= i < len(order)]}, GPU's there "
                      f"{[round(float(glc[order[i]]), 5) for i in (k - 1, k) if 0 <= i < len(order)]}; rank band "
                      f"{rank_m:.3g}; largest GPU log-conf deviation {rep.gpu_lc_dev:.3g})")
        rep.problems.append(f"commit sets differ at decisive positions {where}{detail}")
    both = g_set & o_set
    rep.token_decisions += int(both.sum())
    decisive_tok = both & (tm > tok_m) & ~ex
    rep.exempt_tokens += int((both & ~decisive_tok).sum())
    wrong = decisive_tok & (gpu_after != oracle_after)
    if np.any(wrong):
        rep.problems.append(f"committed tokens differ at {np.nonzero(wrong)[0][:10].tolist()}")
