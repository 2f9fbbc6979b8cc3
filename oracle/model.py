"""Oracle transformer for block-diffusion denoising.  TEST INFRASTRUCTURE ONLY.

What is computed, and where it comes from (page titles abbreviated as
"What changes" = "Diffusion LLMs: what changes when you stop generating one
token at a time"; "DiffusionGemma 4x" = "DiffusionGemma: 4x Faster Text
Generation via Parallel Diffusion"):

  * A Transformer reads the partly masked block and predicts tokens at masked
    positions (What changes, section 2, reverse process).
  * Attention inside the block is bidirectional: every canvas token attends to
    every other canvas token (What changes, section 2, property 1;
    DiffusionGemma 4x, "Bi-directional Attention").
  * Prefill is causal; denoising is bidirectional; finished canvases are appended
    to the KV cache (What changes, section 4.2, "Block decoding").  Blocks are
    autoregressive across, diffusion within (What changes, section 4.1).
  * The FFN of the 26B model is a mixture of experts (What changes, section 4.2;
    DiffusionGemma 4x, "Parallel Generation and Hardware Efficiency").

The pages give no layer internals.  The readings taken here (pre-RMSNorm
blocks, rotate-half RoPE at absolute positions, SwiGLU, softmax-then-top-k
routing renormalised over the chosen experts, an ungated shared expert, untied
LM head, [MASK] excluded from the prediction, confidence = max softmax
probability) are the plainest ones consistent with the pages and the workload
definitions.

Arithmetic is float64.  Values the model stores in a narrower format are rounded
at the point of storage (see `Precision`).

Parity status: rms/softmax/attention/rope/swiglu/moe are pinned by the tests in
tests/test_oracle_*.py (brute force, library routines, closed forms,
invariants).  The composition into a whole model is pinned by the KV-cache
equivalences and the perturbation tests; whole-model logits have no printed
values on the pages to pin against ("parity unpinned" beyond those).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .numerics import e4m3_decode, mxfp4_decode, mxfp6_decode, quant_per_token_e4m3, round_bf16

NEG_INF = -np.inf


# ---------------------------------------------------------------- primitives --

def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(s - max) / sum(exp(s - max)); -inf entries get probability 0."""
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def rope(v: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotary embedding, rotate-half pairing.

    v: [n, heads, dh]; pos: [n] absolute positions.  For i < dh/2 the pair
    (v[i], v[i + dh/2]) is rotated by the angle pos * base**(-2i/dh).
    """
    n, _, dh = v.shape
    half = dh // 2
    theta = base ** (-2.0 * np.arange(half) / dh)                # [half]
    ang = pos.astype(np.float64)[:, None] * theta[None, :]        # [n, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = v[..., :half], v[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Grouped-query attention softmax(q k^T / sqrt(dh)) v.

    q: [Hq, n, dh]; k, v: [Hkv, m, dh]; allowed: [n, m] bool (True = key
    visible).  Query head h reads KV head h // (Hq / Hkv).  Returns [Hq, n, dh].
    """
    hq, n, dh = q.shape
    group = hq // k.shape[0]
    out = np.empty_like(q)
    for h in range(hq):
        s = q[h] @ k[h // group].T / np.sqrt(dh)
        s = np.where(allowed, s, NEG_INF)
        out[h] = softmax(s) @ v[h // group]
    return out


def causal_mask(q_pos: np.ndarray, n_keys: int) -> np.ndarray:
    """Prefill: the query at absolute position p sees keys 0..p."""
    return np.arange(n_keys)[None, :] <= q_pos[:, None]


def block_mask(n_queries: int, n_keys: int) -> np.ndarray:
    """Denoising: every canvas query sees the whole prefix and the whole canvas."""
    return np.ones((n_queries, n_keys), dtype=bool)


# ------------------------------------------------------------------ weights --

class OracleWeights:
    """float64 views of the stored weights.  fp8 projections are kept as the
    decoded E4M3 values plus their per-output-channel fp32 scales."""

    def __init__(self, cfg, tensors: Dict[str, "object"]):
        import torch  # only for reading the synth tensors

        self.cfg = cfg
        self.w: Dict[str, np.ndarray] = {}
        self.s: Dict[str, np.ndarray] = {}
        for name, t in tensors.items():
            if name.endswith(".q"):
                base = name[:-2]
                self.w[base] = e4m3_decode(t.detach().cpu().numpy())
            elif name.endswith(".s"):
                self.s[name[:-2]] = t.detach().to("cpu", torch.float64).numpy()
            elif name.endswith(".q4"):
                # MXFP4: two E2M1 codes per byte (element 2i low nibble), E8M0 block scales
                packed = t.detach().cpu().numpy()
                codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(*packed.shape[:-1], -1)
                self.w[name[:-3]] = mxfp4_decode(codes, tensors[name[:-3] + ".e8"].detach().cpu().numpy())
            elif name.endswith(".q6"):
                # MXFP6 (E2M3): four 6-bit codes per 3 bytes (element 4i + j at bits
                # 6j of the little-endian 24-bit group i), E8M0 block scales
                b = t.detach().cpu().numpy().astype(np.uint32)
                g = b.reshape(*b.shape[:-1], -1, 3)
                bits = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
                codes = np.stack([(bits >> (6 * j)) & 63 for j in range(4)], axis=-1).reshape(*b.shape[:-1], -1)
                self.w[name[:-3]] = mxfp6_decode(codes.astype(np.uint8),
                                                 tensors[name[:-3] + ".e8"].detach().cpu().numpy())
            elif name.endswith(".e8"):
                pass
            else:
                self.w[name] = t.detach().to("cpu", torch.float64).numpy()

    def __getitem__(self, name: str) -> np.ndarray:
        return self.w[name]

    def scale(self, name: str) -> Optional[np.ndarray]:
        return self.s.get(name)


@dataclass
class Precision:
    """Where the model rounds.  f32 models keep every value exact (the oracle's
    float64 stands for the GPU's fp32).  bf16 and fp8 models store GEMM
    A-operands, Q/K/V, the KV cache and the attention output in bf16; fp8 models
    then quantise each GEMM A-operand per token to E4M3 from its bf16 value."""
    dtype: str

    def store(self, x: np.ndarray) -> np.ndarray:
        return x if self.dtype == "f32" else round_bf16(x)


# --------------------------------------------------------------- the model --

@dataclass
class SeqState:
    """One request: KV cache per layer ([Hkv, capacity, dh] each for K and V) and
    the number of cached tokens T."""
    k: List[np.ndarray]
    v: List[np.ndarray]
    T: int = 0


@dataclass
class StepDebug:
    logits: Optional[np.ndarray] = None          # [C, V] with mask column = -inf
    router_sets: List[np.ndarray] = field(default_factory=list)   # per layer [C, k]
    router_gap: List[np.ndarray] = field(default_factory=list)    # per layer [C] k-th minus (k+1)-th logit
    router_logits: List[np.ndarray] = field(default_factory=list)  # per layer [C, E]


class OracleModel:
    """`perturb`: None for the model itself.  The parity tests set it to a
    function y -> y' to measure how far the model's own outputs move when every
    contraction result (GEMM outputs, router logits, attention outputs) carries
    a relative error of fp32 accumulation size; it is applied before the result
    is stored or rounded, and changes nothing else."""

    def __init__(self, cfg, weights: OracleWeights):
        self.cfg = cfg
        self.W = weights
        self.p = Precision(cfg.dtype)
        self.perturb = None

    def _contract(self, y: np.ndarray) -> np.ndarray:
        return y if self.perturb is None else self.perturb(y)

    # -- state
    def new_seq(self, capacity: int) -> SeqState:
        c = self.cfg
        shape = (c.n_kv_heads, capacity, c.head_dim)
        return SeqState([np.zeros(shape) for _ in range(c.n_layers)],
                        [np.zeros(shape) for _ in range(c.n_layers)], 0)

    # -- linear layers
    def linear(self, x: np.ndarray, name: str, w: Optional[np.ndarray] = None,
               s_out: Optional[np.ndarray] = None) -> np.ndarray:
        """y = A W^T with the GEMM A-operand stored as the model declares:
        exact (f32), bf16, or bf16 then per-token E4M3 with
        y = (sum q*w_q) * s_token * s_channel (fp8)."""
        w = self.W[name] if w is None else w
        if self.cfg.dtype == "f32":
            return self._contract(x @ w.T)
        a = round_bf16(x)
        if self.cfg.dtype == "bf16":
            return self._contract(a @ w.T)
        s_o = self.W.scale(name) if s_out is None else s_out
        q, s_t = quant_per_token_e4m3(a)
        return self._contract((q @ w.T) * s_t[:, None] * s_o[None, :])

    def swiglu(self, h: np.ndarray, gate: str, up: str, down: str,
               e: Optional[int] = None) -> np.ndarray:
        """W_down (silu(W_gate h) * (W_up h))."""
        if e is None:
            g, u = self.linear(h, gate), self.linear(h, up)
            return self.linear(silu(g) * u, down)
        W, S = self.W, self.W.scale
        g = self.linear(h, gate, W[gate][e], None if S(gate) is None else S(gate)[e])
        u = self.linear(h, up, W[up][e], None if S(up) is None else S(up)[e])
        return self.linear(silu(g) * u, down, W[down][e], None if S(down) is None else S(down)[e])

    def router(self, h: np.ndarray, l: int):
        """Softmax over all experts of r = h W_r^T (bf16 operands, fp32 logits),
        then the top_k experts (ties to the lower expert id), their
        probabilities renormalised to sum to 1."""
        c = self.cfg
        r = self._contract(self.p.store(h) @ self.W[f"{l}.w_router"].T)   # [n, E]
        p = softmax(r)
        order = np.argsort(-p, axis=-1, kind="stable")              # ties -> lower id first
        sel = order[:, : c.top_k]
        ps = np.take_along_axis(p, sel, axis=-1)
        w = ps / ps.sum(axis=-1, keepdims=True)
        rs = np.take_along_axis(r, order, axis=-1)
        gap = rs[:, c.top_k - 1] - rs[:, c.top_k] if c.top_k < c.n_experts else np.full(len(r), np.inf)
        return sel, w, gap, r

    def moe(self, h: np.ndarray, l: int, dbg: Optional[StepDebug] = None) -> np.ndarray:
        """sum over the chosen experts of weight * SwiGLU_e(h), plus the ungated
        shared SwiGLU(h)."""
        p = f"{l}."
        sel, w, gap, logits = self.router(h, l)
        if dbg is not None:
            dbg.router_sets.append(np.sort(sel, axis=-1))
            dbg.router_gap.append(gap)
            dbg.router_logits.append(logits)
        y = self.swiglu(h, p + "w_gate", p + "w_up", p + "w_down")
        for e in range(self.cfg.n_experts):
            rows, slots = np.nonzero(sel == e)
            if len(rows) == 0:
                continue
            ye = self.swiglu(h[rows], p + "we_gate", p + "we_up", p + "we_down", e=e)
            y[rows] += w[rows, slots][:, None] * ye
        return y

    # -- one transformer block
    def layer(self, l: int, x: np.ndarray, st: SeqState, causal: bool,
              dbg: Optional[StepDebug] = None) -> np.ndarray:
        c, p = self.cfg, f"{l}."
        n = x.shape[0]
        pos = np.arange(st.T, st.T + n)
        h = rms_norm(x, self.W[p + "attn_norm"], c.rms_eps)
        q = self.linear(h, p + "wq").reshape(n, c.n_q_heads, c.head_dim)
        k = self.linear(h, p + "wk").reshape(n, c.n_kv_heads, c.head_dim)
        v = self.linear(h, p + "wv").reshape(n, c.n_kv_heads, c.head_dim)
        q = self.p.store(rope(q, pos, c.rope_base))
        k = self.p.store(rope(k, pos, c.rope_base))
        v = self.p.store(v)
        # K/V of these positions go into the cache at [T, T+n)
        st.k[l][:, st.T:st.T + n] = k.transpose(1, 0, 2)
        st.v[l][:, st.T:st.T + n] = v.transpose(1, 0, 2)
        n_keys = st.T + n
        allowed = causal_mask(pos, n_keys) if causal else block_mask(n, n_keys)
        o = attention(q.transpose(1, 0, 2), st.k[l][:, :n_keys], st.v[l][:, :n_keys], allowed)
        o = self.p.store(self._contract(o.transpose(1, 0, 2).reshape(n, c.q_dim)))
        x = x + self.linear(o, p + "wo")
        h2 = rms_norm(x, self.W[p + "ffn_norm"], c.rms_eps)
        if c.ffn == "dense":
            x = x + self.swiglu(h2, p + "w_gate", p + "w_up", p + "w_down")
        else:
            x = x + self.moe(h2, l, dbg)
        return x

    def forward(self, ids: np.ndarray, st: SeqState, causal: bool,
                dbg: Optional[StepDebug] = None) -> np.ndarray:
        x = self.W["embed"][np.asarray(ids, dtype=np.int64)].copy()
        for l in range(self.cfg.n_layers):
            x = self.layer(l, x, st, causal, dbg)
        return x

    # -- the four operations
    def prefill(self, st: SeqState, ids: np.ndarray, dbg: Optional[StepDebug] = None) -> None:
        """Causal forward over ids at positions [T, T+n); K/V cached; T += n.
        No LM head.  `dbg` (optional) records the routing of every layer."""
        self.forward(ids, st, causal=True, dbg=dbg)
        st.T += len(ids)

    def logits(self, x: np.ndarray) -> np.ndarray:
        h = rms_norm(x, self.W["final_norm"], self.cfg.rms_eps)
        return self.linear(h, "lm_head")

    def denoise(self, st: SeqState, canvas: np.ndarray, debug: bool = False):
        """One denoising pass over the canvas at positions [T, T+C), attending
        to the cached prefix and bidirectionally within the canvas.  The canvas'
        K/V are written at [T, T+C) as scratch; T does not advance.

        Returns (conf, pred, dbg): pred = lowest-id argmax of the logits over the
        vocabulary without [MASK]; conf = max softmax probability over the same
        set = 1 / sum exp(l - max).
        """
        dbg = StepDebug() if debug else None
        x = self.forward(canvas, st, causal=False, dbg=dbg)
        lg = self.logits(x)
        lg[:, self.cfg.mask_id] = NEG_INF
        m = lg.max(axis=-1)
        pred = np.argmax(lg, axis=-1).astype(np.int32)   # first maximum = lowest id
        z = np.exp(lg - m[:, None]).sum(axis=-1)
        conf = 1.0 / z
        if dbg is not None:
            dbg.logits = lg
        return conf, pred, dbg

    def append(self, st: SeqState, canvas: np.ndarray, dbg: Optional[StepDebug] = None) -> None:
        """Forward over the finished canvas with the denoising mask, writing its
        K/V at [T, T+C); then T += C.  No LM head.  `dbg` (optional) records
        the routing of every layer."""
        self.forward(canvas, st, causal=False, dbg=dbg)
        st.T += len(canvas)
