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
midpoint, and for saturation.  The OCP Microscaling (MX v1.0) element formats
E2M1 (MXFP4) and E2M3 (MXFP6): the value tables against the specification's,
rounding by brute force over the representable values, the block quantisers'
shared exponents, error bounds and round trips (tests/test_oracle_mxfp4.py).
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float(np.ldexp(2.0 - 2.0 ** -7, 127))
E4M3_MAX = 448.0


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even (8 significant bits,
    exponent range of fp32, subnormals kept, overflow to +-inf)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    # bf16's normal range: keep the 8 leading significant bits of the float64
    # value (1 implicit + 7 of its 52 fraction bits) and round the 45 bits below
    # them to nearest, ties to the even kept pattern; a carry out of the
    # fraction moves the exponent up, as rounding does
    b = x.view(np.uint64)
    rb = b >> np.uint64(45)
    rb &= np.uint64(1)
    rb += np.uint64((1 << 44) - 1)
    rb += b
    rb &= ~np.uint64((1 << 45) - 1)
    r = rb.view(np.float64)
    ax = np.abs(x)
    if not (np.isfinite(ax).all() and ax.max(initial=0.0) < BF16_MAX and
            ax[ax != 0].min(initial=np.inf) >= 2.0 ** -126):
        r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, x), r)
        # below 2**-126 bf16 values are multiples of 2**-133 (scaling by 2**133 is exact)
        tiny = ax < 2.0 ** -126
        r = np.where(tiny, np.round(x * 2.0 ** 133) * 2.0 ** -133, r)
        r = np.where(np.isfinite(x), r, x)
    return r


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


# ----------------------------------------------------------------- MXFP4 --
# OCP Microscaling Formats (MX) v1.0: an MXFP4 block is 32 consecutive
# elements in FP4 E2M1 sharing one E8M0 scale.  The pages name a 4-bit weight
# format for the 26B model's deployment ("DiffusionGemma: 4x Faster Text
# Generation via Parallel Diffusion", "Deployment and Tooling"); MXFP4 is the
# 4-bit block format of this hardware's matrix cores.

MX_BLOCK = 32
E2M1_MAX = 6.0
E2M1_EMAX = 2          # exponent of the largest normal E2M1 value (6 = 1.5 * 2^2)


def e2m1_decode_table() -> np.ndarray:
    """Value of each of the 16 E2M1 codes: sign bit 3, exponent bits 2..1 with
    bias 1, mantissa bit 0; exponent field 0 holds the subnormal m * 0.5; no
    infinity or NaN."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = -1.0 if code & 8 else 1.0
        e, m = (code >> 1) & 3, code & 1
        vals[code] = s * (0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1))
    return vals


_E2M1_TABLE = e2m1_decode_table()


def e8m0_decode(e) -> np.ndarray:
    """E8M0 scale code: 2^(e - 127); the code 255 is NaN."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.ldexp(1.0, e - 127))


def e2m1_round(x) -> np.ndarray:
    """Nearest E2M1 value, ties to the even mantissa, saturating at +-6.  The
    representable magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} lie on a grid of
    spacing 0.5 below 2, 1 in [2, 4) and 2 in [4, 6]; on each grid the even
    multiples are exactly the codes with an even mantissa."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E2M1_MAX, E2M1_MAX)
    a = np.abs(x)
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    return np.copysign(np.round(a / step) * step, x)


def e2m1_encode(x) -> np.ndarray:
    """Codes of e2m1_round(x) (zero keeps the sign of x)."""
    v = e2m1_round(x)
    idx = np.searchsorted(_E2M1_TABLE[:8], np.abs(v))
    return np.where(np.signbit(v), idx | 8, idx).astype(np.uint8)


def mxfp4_quantize(w: np.ndarray):
    """MXFP4 quantisation of the last axis (a multiple of 32): per block of 32
    the shared exponent is floor(log2(max |w|)) - 2, clamped to E8M0's
    [-127, 127] (an all-zero block takes exponent 0), and each element is
    e2m1_round(w / 2^exponent).  Returns (E2M1 codes uint8 with w's shape,
    E8M0 scale codes uint8 [..., K / 32])."""
    w = np.asarray(w, dtype=np.float64)
    blocks = w.reshape(*w.shape[:-1], w.shape[-1] // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))       # amax = f * 2^e, 0.5 <= f < 1
    shared = np.where(amax > 0, e - 1 - E2M1_EMAX, 0)     # floor(log2 amax) = e - 1
    shared = np.clip(shared, -127, 127)
    codes = e2m1_encode(blocks / np.ldexp(1.0, shared)[..., None])
    return codes.reshape(w.shape), (shared + 127).astype(np.uint8)


def mxfp4_decode(codes, scales) -> np.ndarray:
    """Values of MXFP4 data: E2M1 codes [..., K] times their blocks' E8M0 scales
    [..., K / 32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    v = _E2M1_TABLE[codes]
    s = e8m0_decode(scales)
    return (v.reshape(*v.shape[:-1], -1, MX_BLOCK) * s[..., None]).reshape(v.shape)


# ---- MXFP6 (OCP Microscaling v1.0, E2M3 elements) ------------------------------
E2M3_MAX = 7.5
E2M3_EMAX = 2          # exponent of the largest normal E2M3 value (7.5 = 1.875 * 2^2)


def e2m3_decode_table() -> np.ndarray:
    """Value of each of the 64 E2M3 codes: sign bit 5, exponent bits 4..3 with
    bias 1, mantissa bits 2..0; exponent field 0 holds the subnormal m / 8; no
    infinity or NaN."""
    vals = np.empty(64, dtype=np.float64)
    for code in range(64):
        sgn = -1.0 if code & 32 else 1.0
        e, m = (code >> 3) & 3, code & 7
        vals[code] = sgn * (m / 8.0 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 1))
    return vals


_E2M3_TABLE = e2m3_decode_table()


def e2m3_round(x) -> np.ndarray:
    """Nearest E2M3 value, ties to the even mantissa, saturating at +-7.5.  The
    magnitudes lie on a grid of spacing 1/8 below 2 (subnormals and exponent
    1), 1/4 in [2, 4) and 1/2 in [4, 7.5]; on each grid the even multiples are
    the codes with an even mantissa."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E2M3_MAX, E2M3_MAX)
    a = np.abs(x)
    step = np.where(a < 2.0, 0.125, np.where(a < 4.0, 0.25, 0.5))
    return np.copysign(np.round(a / step) * step, x)


def e2m3_encode(x) -> np.ndarray:
    """Codes of e2m3_round(x) (zero keeps the sign of x)."""
    v = e2m3_round(x)
    idx = np.searchsorted(_E2M3_TABLE[:32], np.abs(v))
    return np.where(np.signbit(v), idx | 32, idx).astype(np.uint8)


def mxfp6_quantize(w: np.ndarray):
    """MXFP6 (E2M3) quantisation of the last axis (a multiple of 32): per block
    of 32 the shared exponent is floor(log2(max |w|)) - 2, clamped to E8M0's
    [-127, 127] (an all-zero block takes exponent 0), and each element is
    e2m3_round(w / 2^exponent).  Returns (E2M3 codes uint8 with w's shape,
    E8M0 scale codes uint8 [..., K / 32])."""
    w = np.asarray(w, dtype=np.float64)
    blocks = w.reshape(*w.shape[:-1], w.shape[-1] // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.clip(np.where(amax > 0, e - 1 - E2M3_EMAX, 0), -127, 127)
    codes = e2m3_encode(blocks / np.ldexp(1.0, shared)[..., None])
    return codes.reshape(w.shape), (shared + 127).astype(np.uint8)


def mxfp6_decode(codes, scales) -> np.ndarray:
    """Values of MXFP6 (E2M3) data: codes [..., K] times their blocks' E8M0
    scales [..., K / 32]."""
    codes = np.asarray(codes, dtype=np.uint8)
    v = _E2M3_TABLE[codes]
    s = e8m0_decode(scales)
    return (v.reshape(*v.shape[:-1], -1, MX_BLOCK) * s[..., None]).reshape(v.shape)
