"""GPU kernel-level parity through the C ABI's test entry points."""
import numpy as np
import pytest
import torch

from oracle.numerics import e4m3_decode, quant_per_token_e4m3

pytestmark = pytest.mark.gpu


def _bf16_rows():
    """Rows covering every finite bf16 bit pattern.  Row E holds every value
    (both signs) with a binary exponent in [E - 10, E], plus one element equal
    to 448 * 2^(E + 1 - 8), which makes the row scale an exact power of two so
    that every quotient is exact and halfway cases between E4M3 values occur;
    a second row per E has no such element (scale = amax / 448 not a power of
    two: the division path).  Returns uint16 bit patterns [rows, d]."""
    rows = []
    for E in range(-133, 128):
        vals = []
        for e in range(E - 10, E + 1):
            if e < -133 or e > 127:
                continue
            for m in range(128):
                if e == -133:                      # subnormals 2^-133 .. : mantissa only
                    bits = m
                elif e < -126:
                    continue
                else:
                    bits = ((e + 127) << 7) | m
                if bits == 0 or (bits >> 7) == 0xFF:
                    continue
                vals.append(bits)
                vals.append(bits | 0x8000)
        if not vals:
            continue
        rows.append(vals)
    d = max(len(r) for r in rows) + 1
    out = []
    for r in rows:
        out.append(r + [0] * (d - len(r)))         # scale = amax / 448 (division path)
        amax_bits = max(v & 0x7FFF for v in r)
        E = (amax_bits >> 7) - 127
        exact = np.float32(448.0 * 2.0 ** (E + 1 - 8))
        b = int(np.frombuffer(exact.tobytes(), dtype=np.uint32)[0] >> 16)
        if (b >> 7) & 0xFF != 0xFF:
            out.append(r + [b] * (d - len(r)))     # scale = 2^(E + 1 - 8) exactly
    out.append([0] * d)                            # all-zero row: scale 1
    return np.array(out, dtype=np.uint16)


def test_quant_rows_exhaustive_bf16():
    import ctypes
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    bits = _bf16_rows()
    rows, d = bits.shape
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    q = torch.empty((rows, d), dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    abi.check(lib.dlm_op_quant_rows(x.data_ptr(), rows, d, q.data_ptr(), s.data_ptr(), st), "quant")
    torch.cuda.synchronize()
    xv = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q_o, s_o = quant_per_token_e4m3(xv)
    g_codes = q.cpu().numpy()
    g_s = s.cpu().numpy().astype(np.float64)
    assert np.array_equal(g_s, s_o), f"scales differ in {np.sum(g_s != s_o)} rows"
    g_vals = e4m3_decode(g_codes)
    bad = g_vals != q_o
    assert not np.any(bad), (f"{bad.sum()} codes differ, e.g. x={xv[bad][:4]}, gpu={g_vals[bad][:4]}, "
                             f"oracle={q_o[bad][:4]}")
    assert not np.any(g_codes == 0x7F) and not np.any(g_codes == 0xFF), "NaN code produced"
    print(f"[ops] quantised {rows} x {d} bf16 values bit-exactly", flush=True)


def test_quant_rows_rejects_bad_args():
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    assert lib.dlm_op_quant_rows(None, 1, 1, None, None, None) == abi.DLM_E_ARG
    x = torch.zeros(4, dtype=torch.bfloat16, device="cuda")
    assert lib.dlm_op_quant_rows(x.data_ptr(), 0, 4, x.data_ptr(), x.data_ptr(), None) == abi.DLM_E_ARG
