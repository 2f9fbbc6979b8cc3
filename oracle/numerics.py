"""Storage rounding used by the oracle: bf16 and OCP FP8 E4M3FN.  TEST INFRASTRUCTURE.

The pages fix no number format beyond "FP8" for the H100 measurement (Diffusion
LLMs: what changes..., section 4.2, speed bullet).  The model precisions are the
workload definitions': bf16 storage with fp32 accumulation, and fp8 E4M3 with
per-output-channel weight scales and per-token dynamic activation scales.

The oracle computes in float64 and rounds values to the storage format at the
points where the model stores them.  Rounding is done directly from the float64
value (no intermediate fp32 rounding).

Pins: round_bf16 against torch's fp32->bf16 conversion over fp32 bit patterns;
e4m3_decode against the format's definition for all 256 codes and against
torch.float8_e4m3fn; e4m3_encode against torch on in-range values, at every
midpoint, and for saturation.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float(np.ldexp(2.0 - 2.0 ** -7, 127))
E4M3_MAX = 448.0


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even (8 significant bits,
    exponent range of fp32, subnormals kept, overflow to +-inf)."""
    x = np.asarray(x, dtype=np.float64)
    finite = np.isfinite(x) & (x != 0)
    out = x.copy()
    xf = x[finite]
    _, e = np.frexp(xf)                 # xf = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)             # below 2**-126 the spacing stays 2**-133
    ulp = np.ldexp(1.0, e - 8)
    r = np.round(xf / ulp) * ulp        # np.round: half to even; xf/ulp is exact
    r[np.abs(r) > BF16_MAX] = np.inf * np.sign(r[np.abs(r) > BF16_MAX])
    out[finite] = r
    return out


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (OCP 8-bit floating point spec):
    sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0
    holds subnormals m/8 * 2**-6; S.1111.111 is NaN; there is no infinity."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        ef = (code >> 3) & 0xF
        mf = code & 0x7
        if ef == 0xF and mf == 0x7:
            vals[code] = np.nan
        elif ef == 0:
            vals[code] = s * (mf / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + mf / 8.0) * 2.0 ** (ef - 7)
    return vals


_E4M3_TABLE = e4m3_decode_table()


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3FN value, ties to even, saturating at +-448 (no NaN for
    finite inputs)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    xf = np.clip(x[nz], -E4M3_MAX, E4M3_MAX)
    _, e = np.frexp(xf)
    e = np.maximum(e, -5)               # min normal 2**-6 = 0.5 * 2**-5
    ulp = np.ldexp(1.0, e - 4)          # 4 significant bits
    r = np.round(xf / ulp) * ulp
    out[nz] = np.clip(r, -E4M3_MAX, E4M3_MAX)
    return out


def e4m3_encode(x) -> np.ndarray:
    """Codes of e4m3_round(x)."""
    v = e4m3_round(x)
    pos = _E4M3_TABLE[:0x7F]            # non-negative finite codes 0x00..0x7E, ascending
    idx = np.searchsorted(pos, np.abs(v))
    codes = idx.astype(np.uint8)
    codes = np.where(v < 0, codes | 0x80, codes).astype(np.uint8)
    codes = np.where(v == 0, np.uint8(0), codes)
    return codes


def f32(x) -> np.ndarray:
    """Round to IEEE binary32 (values the model holds in fp32)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def quant_per_token_e4m3(x):
    """Per-token (per-row) dynamic E4M3 quantisation of an activation matrix.

    The row's amax and the scale amax/448 are taken in fp32 (the activation is
    held in fp32 before quantisation); a zero row gets scale 1.  The quotient
    x/scale is formed in fp32 with IEEE division, then rounded to E4M3 with ties
    to even and saturation.  Returns (dequantisation-ready values q in float64,
    scales in float64) so that x ~= q * scale[:, None].
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    amax = np.abs(x32).max(axis=-1)
    s = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32), np.float32(1.0))
    quot = (x32 / s[..., None]).astype(np.float32)
    q = e4m3_round(quot.astype(np.float64))
    return q, s.astype(np.float64)
