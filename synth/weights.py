"""Seeded synthetic weights and inputs.

Random-init weights stand in for trained ones (the pages ship none): every matrix
and embedding is drawn N(0, init_std) (the LM head N(0, lm_head_std) when a
workload sets it, for confidences far from uniform); RMSNorm gains are 1; the router matrix is
drawn N(0, d_model^-1/2) so that router logits have unit variance.  Each tensor
has its own generator, seeded from (run seed, tensor name), so any tensor can be
regenerated alone.  Values are drawn in fp32 and stored in the model's precision:
fp32, bf16 (round-to-nearest-even, by torch's conversion), or for fp8 models
OCP E4M3FN codes with one fp32 scale per output channel, scale = amax / 448.

This module is plumbing shared by the oracle's tests and the HIP path's callers:
it holds no step of the denoising method.  A tensor generated on one device and
the same tensor generated on another are NOT the same draw; callers that compare
the two paths generate once and copy.
"""
from __future__ import annotations

import hashlib
from typing import Dict, List

import torch

from .configs import ModelConfig, RunConfig

E4M3_MAX = 448.0


def tensor_seed(seed: int, name: str) -> int:
    h = hashlib.blake2b(f"{seed}/{name}".encode(), digest_size=8).digest()
    return int.from_bytes(h, "little") & 0x7FFF_FFFF_FFFF_FFFF


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(tensor_seed(seed, name))
    return g


def normal(seed: int, name: str, shape, std: float, device="cpu") -> torch.Tensor:
    g = _gen(seed, name, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x.mul_(std)


def quantize_e4m3_rows(w: torch.Tensor):
    """Per-output-channel (last-dim rows) E4M3FN quantisation of fp32 weights.

    Returns (codes uint8 with the same shape, scales fp32 of shape w.shape[:-1]).
    scale = amax/448 (1 when a row is all zero); code = e4m3(w/scale), round to
    nearest even, saturating at +-448.
    """
    amax = w.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (w / s.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), s.contiguous()


E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)    # codes 0..7; bit 3 is the sign


def quantize_mxfp4_rows(w: torch.Tensor):
    """MXFP4 (OCP Microscaling v1.0) quantisation along the last axis, a
    multiple of 32: each block of 32 shares the E8M0 exponent floor(log2 max|w|)
    - 2 (clamped to [-127, 127]; 0 for an all-zero block) and each element is
    w / 2^exponent rounded to the nearest E2M1 value, ties to the even
    mantissa, saturating at +-6.

    Returns (codes uint8 [..., K / 2], two E2M1 codes per byte, element 2i in
    the low nibble and 2i + 1 in the high one; scales uint8 [..., K / 32],
    the E8M0 codes exponent + 127)."""
    blocks = w.float().reshape(*w.shape[:-1], w.shape[-1] // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, e = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))   # amax = m * 2^e, m in [0.5, 1)
    shared = torch.where(amax > 0, e - 3, torch.zeros_like(e)).clamp_(-127, 127)
    x = torch.ldexp(blocks, -shared.unsqueeze(-1).float())
    a = x.abs().clamp_(max=6.0)
    step = torch.where(a < 2.0, 0.5, torch.where(a < 4.0, 1.0, 2.0))
    r = torch.round(a / step) * step                                          # half to even on each grid
    mags = torch.tensor(E2M1_MAGNITUDES, dtype=r.dtype, device=r.device)
    codes = torch.bucketize(r, mags).to(torch.uint8) | (torch.signbit(x).to(torch.uint8) << 3)
    codes = codes.reshape(w.shape)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed.contiguous(), (shared + 127).to(torch.uint8).contiguous()


E2M3_MAGNITUDES = tuple([m / 8 for m in range(8)] + [1 + m / 8 for m in range(8)] + [2 + m / 4 for m in range(8)]
                        + [4 + m / 2 for m in range(8)])    # codes 0..31; bit 5 is the sign


def quantize_mxfp6_rows(w: torch.Tensor):
    """MXFP6 with E2M3 elements (OCP Microscaling v1.0) along the last axis, a
    multiple of 32: each block of 32 shares the E8M0 exponent floor(log2
    max|w|) - 2 (clamped to [-127, 127]; 0 for an all-zero block) and each
    element is w / 2^exponent rounded to the nearest E2M3 value, ties to the
    even mantissa, saturating at +-7.5.

    Returns (codes uint8 [..., K * 3 / 4]: four 6-bit codes per 3 bytes,
    element 4i + j at bits 6j .. 6j + 5 of the little-endian 24-bit group i;
    scales uint8 [..., K / 32], the E8M0 codes exponent + 127)."""
    blocks = w.float().reshape(*w.shape[:-1], w.shape[-1] // 32, 32)
    amax = blocks.abs().amax(dim=-1)
    _, e = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
    shared = torch.where(amax > 0, e - 3, torch.zeros_like(e)).clamp_(-127, 127)
    x = torch.ldexp(blocks, -shared.unsqueeze(-1).float())
    a = x.abs().clamp_(max=7.5)
    step = torch.where(a < 2.0, 0.125, torch.where(a < 4.0, 0.25, 0.5))
    r = torch.round(a / step) * step                                          # half to even on each grid
    mags = torch.tensor(E2M3_MAGNITUDES, dtype=r.dtype, device=r.device)
    codes = torch.bucketize(r, mags).to(torch.int32) | (torch.signbit(x).to(torch.int32) << 5)
    g = codes.reshape(*w.shape[:-1], w.shape[-1] // 4, 4)
    bits = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
    packed = torch.stack([bits & 255, (bits >> 8) & 255, (bits >> 16) & 255], dim=-1).to(torch.uint8)
    return packed.reshape(*w.shape[:-1], w.shape[-1] * 3 // 4).contiguous(), (shared + 127).to(torch.uint8).contiguous()


def _store(out: Dict[str, torch.Tensor], name: str, w: torch.Tensor, dtype: str,
           projection: bool):
    if dtype == "mxfp6":
        q, e = quantize_mxfp6_rows(w)
        out[name + ".q6"] = q
        out[name + ".e8"] = e
    elif dtype == "mxfp4":
        q, e = quantize_mxfp4_rows(w)
        out[name + ".q4"] = q
        out[name + ".e8"] = e
    elif dtype == "f32":
        out[name] = w.contiguous()
    elif dtype == "bf16" or not projection:
        out[name] = w.to(torch.bfloat16).contiguous()
    elif dtype == "fp8":
        q, s = quantize_e4m3_rows(w)
        out[name + ".q"] = q.contiguous()
        out[name + ".s"] = s
    else:
        raise ValueError(dtype)


def projection_names(cfg: ModelConfig) -> List[str]:
    names = ["wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"]
    if cfg.ffn == "moe":
        names += ["we_gate", "we_up", "we_down"]
    return names


def make_weights(cfg: ModelConfig, seed: int = 0, device="cpu",
                 layers=None) -> Dict[str, torch.Tensor]:
    """All weights of `cfg`, keyed '<name>' or '<layer>.<name>'.

    `layers` restricts generation to a subset of layer indices (the others are
    simply absent), for tests that check one layer at full size.
    """
    d, std = cfg.d_model, cfg.init_std
    out: Dict[str, torch.Tensor] = {}
    emb = normal(seed, "embed", (cfg.vocab, d), std, device)
    out["embed"] = emb.contiguous() if cfg.dtype == "f32" else emb.to(torch.bfloat16).contiguous()
    del emb
    out["final_norm"] = torch.ones(d, dtype=torch.float32, device=device)
    lm_std = std if cfg.lm_head_std is None else cfg.lm_head_std
    _store(out, "lm_head", normal(seed, "lm_head", (cfg.vocab, d), lm_std, device),
           cfg.dtype, projection=True)
    for l in (range(cfg.n_layers) if layers is None else layers):
        p = f"{l}."
        out[p + "attn_norm"] = torch.ones(d, dtype=torch.float32, device=device)
        out[p + "ffn_norm"] = torch.ones(d, dtype=torch.float32, device=device)
        shapes = {
            "wq": (cfg.q_dim, d), "wk": (cfg.kv_dim, d), "wv": (cfg.kv_dim, d),
            "wo": (d, cfg.q_dim),
            "w_gate": (cfg.d_ffn, d), "w_up": (cfg.d_ffn, d), "w_down": (d, cfg.d_ffn),
        }
        if cfg.ffn == "moe":
            E, de = cfg.n_experts, cfg.d_expert
            shapes.update({"we_gate": (E, de, d), "we_up": (E, de, d), "we_down": (E, d, de)})
        for name, shape in shapes.items():
            dt = cfg.expert_dtype if (name.startswith("we_") and cfg.expert_dtype) else cfg.dtype
            _store(out, p + name, normal(seed, p + name, shape, std, device), dt, projection=True)
        if cfg.ffn == "moe":
            wr = normal(seed, p + "w_router", (cfg.n_experts, d), cfg.router_sigma, device)
            out[p + "w_router"] = wr.contiguous() if cfg.dtype == "f32" else wr.to(torch.bfloat16).contiguous()
    return out


def prefix_lengths(run: RunConfig) -> List[int]:
    lo, hi = run.prefix_len
    if lo == hi:
        return [lo] * run.n_requests
    g = _gen(run.seed, "prefix_lengths", "cpu")
    return torch.randint(lo, hi + 1, (run.n_requests,), generator=g).tolist()


def prefix_ids(run: RunConfig, request: int, length: int, device="cpu") -> torch.Tensor:
    """Uniform ids in [0, V-2]: a prompt never holds the [MASK] id (V-1)."""
    g = _gen(run.seed, f"prefix_ids/{request}", device)
    hi = run.model.vocab - 1   # exclusive bound -> ids 0..V-2
    return torch.randint(0, hi, (length,), generator=g, device=device, dtype=torch.int64).to(torch.int32)


def make_inputs(run: RunConfig, device="cpu") -> List[torch.Tensor]:
    return [prefix_ids(run, r, n, device) for r, n in enumerate(prefix_lengths(run))]


def to_float64_numpy(t: torch.Tensor):
    """Exact float64 copy of a stored fp32 or bf16 tensor."""
    return t.detach().to("cpu", torch.float64).numpy()
