"""Pins for the oracle's storage rounding (bf16, OCP E4M3FN)."""
import numpy as np
import pytest
import torch

from oracle.numerics import (E4M3_MAX, e4m3_decode, e4m3_decode_table, e4m3_encode,
                             e4m3_round, quant_per_token_e4m3, round_bf16)


def _fp32_patterns(n, seed=0):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_bf16_matches_torch_on_fp32_patterns():
    x = _fp32_patterns(1 << 22)
    # add the neighbourhood of every rounding boundary class: ties, subnormals, overflow
    edges = np.array([0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 - 2 ** -9,
                      np.float32(3.3895314e38), np.float32(3.4028235e38), 2 ** -126,
                      2 ** -133, 2 ** -134, 3 * 2 ** -134, 1e-40, -1e-42], dtype=np.float32)
    x = np.concatenate([x, edges, -edges])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_bf16_ties_to_even_closed_form():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: the even neighbour is 1
    assert round_bf16(1.0 + 2 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert round_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6
    # just above a tie rounds up (fp64 input, no double rounding)
    assert round_bf16(1.0 + 2 ** -8 + 2 ** -40) == 1.0 + 2 ** -7
    assert round_bf16(-(1.0 + 2 ** -8 + 2 ** -40)) == -(1.0 + 2 ** -7)
    assert np.isinf(round_bf16(3.5e38))


def test_e4m3_table_from_spec():
    t = e4m3_decode_table()
    assert t[0x00] == 0.0 and t[0x38] == 1.0 and t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6          # min normal
    assert t[0x01] == 2.0 ** -9          # min subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # max subnormal
    assert t[0x3C] == 1.5 and t[0x40] == 2.0 and t[0x5C] == 24.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    fin = t[:0x7F]
    assert np.all(np.diff(fin) > 0)


def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = e4m3_decode_table()
    both_nan = np.isnan(tv) & np.isnan(t)
    np.testing.assert_array_equal(t[~both_nan], tv[~both_nan])


def test_e4m3_round_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200_000) * s for s in (1e-3, 0.05, 1, 30, 200)])
    x = np.clip(x, -E4M3_MAX, E4M3_MAX).astype(np.float32)
    # every midpoint between consecutive finite codes (exactly representable in fp32)
    fin = e4m3_decode_table()[:0x7F]
    mids = ((fin[1:] + fin[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(e4m3_round(x.astype(np.float64)), want)


def test_e4m3_ties_and_saturation():
    assert e4m3_round(1.0 + 1 / 16) == 1.0            # tie -> even mantissa 000
    assert e4m3_round(1.0 + 3 / 16) == 1.25           # tie -> even mantissa 010
    assert e4m3_round(1000.0) == 448.0 and e4m3_round(-1e9) == -448.0
    assert e4m3_round(464.0) == 448.0
    assert e4m3_round(2.0 ** -10) == 0.0              # half of min subnormal -> even (0)
    assert e4m3_round(3 * 2.0 ** -10) == 2 * 2.0 ** -9


def test_e4m3_encode_roundtrip():
    t = e4m3_decode_table()
    finite = np.nonzero(~np.isnan(t))[0]
    finite = finite[finite != 0x80]                  # -0 encodes as +0
    np.testing.assert_array_equal(e4m3_encode(t[finite]), finite.astype(np.uint8))
    np.testing.assert_array_equal(e4m3_decode(e4m3_encode([0.3, -7.0, 500.0])),
                                  e4m3_round([0.3, -7.0, 500.0]))


def test_quant_per_token():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 64))
    x[3] = 0.0
    q, s = quant_per_token_e4m3(x)
    assert s[3] == 1.0 and np.all(q[3] == 0)
    for r in (0, 1, 2, 4):
        j = np.argmax(np.abs(x[r]))
        assert abs(q[r, j]) == 448.0                  # the row's amax lands on the top code
        assert s[r] == np.float32(np.float32(np.abs(x[r]).max()) / np.float32(448.0))
    # dequantisation error is within half an E4M3 step (relative 2^-4) of each value
    rel = np.abs(q * s[:, None] - x) / np.maximum(np.abs(x), 2 ** -6 * s[:, None])
    assert rel[[0, 1, 2, 4]].max() <= 2 ** -4 + 1e-6
