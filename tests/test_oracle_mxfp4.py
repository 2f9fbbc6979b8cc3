"""Pins of the oracle's MX functions (oracle/numerics.py) against the OCP
Microscaling (MX) v1.0 format definition: the E2M1 (MXFP4) and E2M3 (MXFP6)
value tables, E8M0 scales, round-to-nearest-even with saturation (brute force
over the representable values), and the block quantisers' shared exponents."""
import numpy as np

from oracle.numerics import (E2M1_MAX, E2M3_MAX, MX_BLOCK, e2m1_decode_table, e2m1_encode, e2m1_round,
                             e2m3_decode_table, e2m3_encode, e2m3_round, e8m0_decode, mxfp4_decode, mxfp4_quantize,
                             mxfp6_decode, mxfp6_quantize)

# the format's value table: codes 0..7 are the non-negative values, 8..15 their negatives
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_is_the_spec_table():
    t = e2m1_decode_table()
    np.testing.assert_array_equal(t[:8], SPEC_E2M1)
    np.testing.assert_array_equal(t[8:], [-v for v in SPEC_E2M1])
    assert np.signbit(t[8]) and t[8] == 0.0


def test_e8m0_scales():
    np.testing.assert_array_equal(e8m0_decode([127, 128, 126, 0, 254]), [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127])
    assert np.isnan(e8m0_decode(255))


def test_e2m1_round_midpoints_and_saturation():
    # every midpoint between neighbours goes to the value with the even mantissa (code bit 0 clear)
    cases = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for x, want in cases.items():
        assert e2m1_round(x) == want and e2m1_round(-x) == -want
        assert e2m1_encode(want) & 1 == 0
    for x in (6.0, 6.5, 7.99, 1e9):
        assert e2m1_round(x) == 6.0 and e2m1_round(-x) == -6.0


def test_e2m1_round_is_the_nearest_value_brute_force():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-7, 7, 20000), np.array(SPEC_E2M1) * 1.0])
    vals = np.array(SPEC_E2M1)
    got = e2m1_round(x)
    a = np.minimum(np.abs(x), E2M1_MAX)
    dist = np.abs(a[:, None] - vals[None, :])
    best = dist.min(axis=1)
    # the result is one of the nearest values (ties are the midpoint cases above)
    assert np.all(np.abs(np.abs(got) - a) <= best + 1e-12)
    assert np.all(np.isin(np.abs(got), vals))


def test_encode_decode_roundtrip_of_every_code():
    t = e2m1_decode_table()
    codes = np.arange(16, dtype=np.uint8)
    np.testing.assert_array_equal(e2m1_encode(t), codes)


def test_block_quantiser_shared_exponent():
    # a block whose largest magnitude is 6 keeps scale 1 (code 127) and its values
    w = np.zeros((1, MX_BLOCK))
    w[0, :8] = SPEC_E2M1
    w[0, 8:16] = [-v for v in SPEC_E2M1]
    codes, scales = mxfp4_quantize(w)
    assert scales.tolist() == [[127]]
    np.testing.assert_array_equal(mxfp4_decode(codes, scales), w)
    # max |w| = 1: exponent floor(log2 1) - 2 = -2, elements divided by 1/4
    w = np.full((1, MX_BLOCK), 0.375)
    w[0, 0] = -1.0
    codes, scales = mxfp4_quantize(w)
    assert scales.tolist() == [[125]]
    np.testing.assert_array_equal(mxfp4_decode(codes, scales)[0, :2], [-1.0, 0.375])
    # max |w| just below 8 * 2^k saturates at 6 * 2^k (the clipping the format defines)
    w = np.full((1, MX_BLOCK), 0.01)
    w[0, 5] = 7.9
    codes, scales = mxfp4_quantize(w)
    assert scales.tolist() == [[127]] and mxfp4_decode(codes, scales)[0, 5] == 6.0
    # an all-zero block: exponent 0, zero codes
    codes, scales = mxfp4_quantize(np.zeros((2, 2 * MX_BLOCK)))
    assert scales.tolist() == [[127, 127], [127, 127]] and not codes.any()


def test_block_quantiser_error_bound_and_roundtrip():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((16, 8 * MX_BLOCK)) * 0.02
    codes, scales = mxfp4_quantize(w)
    deq = mxfp4_decode(codes, scales)
    X = e8m0_decode(scales)[..., None]
    blk = w.reshape(16, 8, MX_BLOCK)
    err = np.abs(deq.reshape(16, 8, MX_BLOCK) - blk)
    a = np.abs(blk) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    # within half a step of the element's grid, or the clipping of the largest elements above 6
    assert np.all((err <= step / 2 * X + 1e-15) | (a > E2M1_MAX))
    # quantising dequantised data gives the same codes and scales back
    c2, s2 = mxfp4_quantize(deq)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(mxfp4_decode(c2, s2), deq)


def test_synth_quantiser_agrees_with_the_oracle():
    """The weight generator's MXFP4 quantiser (synth, torch) writes the codes
    and scales both the GPU and the oracle read; it must be the quantiser
    pinned above: identical codes and scales on normal weights, an all-zero
    block, blocks whose maximum is a power of two or just below one, and
    values at E2M1 midpoints."""
    import torch
    from synth.weights import quantize_mxfp4_rows
    rng = np.random.default_rng(7)
    w = rng.standard_normal((6, 256)) * 0.02
    w[0, :32] = 0.0                                       # all-zero block
    w[1, :32] = rng.choice([-1, 1], 32) * 2.0 ** -5       # max a power of two
    w[1, 32:64] = np.linspace(-0.0624, 0.0624, 32)        # max just below 2^-4
    w[2, :32] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0] * 4) * 2.0 ** -3   # midpoints
    w[2, 31] = 6.0 * 2.0 ** -3
    w = w.astype(np.float32).astype(np.float64)          # the generator quantises fp32 values
    q, e = quantize_mxfp4_rows(torch.from_numpy(w).float())
    q = q.numpy()
    codes = np.empty((w.shape[0], w.shape[1]), dtype=np.uint8)
    codes[:, 0::2] = q & 15
    codes[:, 1::2] = q >> 4
    want_codes, want_scales = mxfp4_quantize(w)
    np.testing.assert_array_equal(codes, want_codes)
    np.testing.assert_array_equal(e.numpy(), want_scales)


# the E2M3 value table of the format (positive half; codes 32..63 are the negatives)
SPEC_E2M3 = [0.0, 0.125, 0.25, 0.375, 0.5, 0.625, 0.75, 0.875,
             1.0, 1.125, 1.25, 1.375, 1.5, 1.625, 1.75, 1.875,
             2.0, 2.25, 2.5, 2.75, 3.0, 3.25, 3.5, 3.75,
             4.0, 4.5, 5.0, 5.5, 6.0, 6.5, 7.0, 7.5]


def test_e2m3_table_is_the_spec_table():
    t = e2m3_decode_table()
    np.testing.assert_array_equal(t[:32], SPEC_E2M3)
    np.testing.assert_array_equal(t[32:], [-v for v in SPEC_E2M3])
    assert np.signbit(t[32]) and E2M3_MAX == SPEC_E2M3[-1]


def test_e2m3_round_is_the_nearest_value_brute_force():
    """Against a search over the 32 magnitudes: nearest value, at a tie the one
    whose code is even (the even mantissa), beyond 7.5 the largest."""
    rng = np.random.default_rng(5)
    mids = [(a + b) / 2 for a, b in zip(SPEC_E2M3[:-1], SPEC_E2M3[1:])]
    x = np.concatenate([rng.uniform(-9, 9, 4000), mids, [-m for m in mids], SPEC_E2M3, [7.6, 100.0, -8.0]])
    mags = np.array(SPEC_E2M3)
    for v in x:
        d = np.abs(mags - abs(v))
        best = np.flatnonzero(d == d.min())
        want = mags[best[0]] if len(best) == 1 else mags[[i for i in best if i % 2 == 0][0]]
        want = min(want, E2M3_MAX) if abs(v) <= E2M3_MAX else E2M3_MAX
        assert e2m3_round(v) == np.copysign(want, v), v
    codes = e2m3_encode(np.array(SPEC_E2M3 + [-v for v in SPEC_E2M3]))
    np.testing.assert_array_equal(e2m3_decode_table()[codes], SPEC_E2M3 + [-v for v in SPEC_E2M3])


def test_mxfp6_block_quantiser():
    # a block whose largest magnitude is 7.5 keeps scale 1 (code 127) and its values
    w = np.zeros((1, MX_BLOCK))
    w[0, :16] = SPEC_E2M3[16:]
    w[0, 16:32] = [-v for v in SPEC_E2M3[:16]]
    codes, scales = mxfp6_quantize(w)
    assert scales.tolist() == [[127]]
    np.testing.assert_array_equal(mxfp6_decode(codes, scales), w)
    # max |w| = 1: exponent -2, a step of 1/32 in the block
    w = np.full((1, MX_BLOCK), 1.0 / 32)
    w[0, 0] = -1.0
    w[0, 1] = 1.0 / 64                          # a tie between 0 and 1/32: to the even code (0)
    codes, scales = mxfp6_quantize(w)
    assert scales.tolist() == [[125]]
    np.testing.assert_array_equal(mxfp6_decode(codes, scales)[0, :3], [-1.0, 0.0, 1.0 / 32])
    # saturation: max |w| just below 8 * 2^k becomes 7.5 * 2^k
    w = np.full((1, MX_BLOCK), 0.01)
    w[0, 3] = 7.9
    codes, scales = mxfp6_quantize(w)
    assert scales.tolist() == [[127]] and mxfp6_decode(codes, scales)[0, 3] == 7.5
    # all-zero blocks: exponent 0, zero codes
    codes, scales = mxfp6_quantize(np.zeros((2, 2 * MX_BLOCK)))
    assert scales.tolist() == [[127, 127], [127, 127]] and not codes.any()
    # error bound: within half the coarsest grid step (0.5 * 2^shared) of the
    # block, except where the block maximum saturates (|w| above 7.5 * 2^shared)
    rng = np.random.default_rng(2)
    w = rng.standard_normal((8, 4 * MX_BLOCK)) * 0.02
    codes, scales = mxfp6_quantize(w)
    q = mxfp6_decode(codes, scales)
    unit = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)        # 2^shared per element
    bound = np.where(np.abs(w) > 7.5 * unit, np.abs(w) - 7.5 * unit, 0.25 * unit)
    assert np.all(np.abs(q - w) <= bound + 1e-18)
    np.testing.assert_array_equal(mxfp6_quantize(q)[0], codes)      # decoded values quantise to themselves


def test_synth_mxfp6_quantiser_agrees_with_the_oracle():
    """The weight generator's MXFP6 quantiser (synth, torch, packed four codes
    per 3 bytes) gives the oracle's codes and scales."""
    import torch
    from synth.weights import quantize_mxfp6_rows
    rng = np.random.default_rng(11)
    w = rng.standard_normal((5, 256)) * 0.02
    w[0, :32] = 0.0
    w[1, :32] = np.array(SPEC_E2M3) * 2.0 ** -4
    w[2, :31] = np.array([(a + b) / 2 for a, b in zip(SPEC_E2M3[:-1], SPEC_E2M3[1:])]) * 2.0 ** -5
    w[2, 31] = 7.5 * 2.0 ** -5
    w = w.astype(np.float32).astype(np.float64)
    q, e = quantize_mxfp6_rows(torch.from_numpy(w).float())
    b = q.numpy().astype(np.uint32).reshape(5, -1, 3)
    bits = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
    codes = np.stack([(bits >> (6 * j)) & 63 for j in range(4)], axis=-1).reshape(5, -1)
    want_codes, want_scales = mxfp6_quantize(w)
    np.testing.assert_array_equal(codes, want_codes)
    np.testing.assert_array_equal(e.numpy(), want_scales)
