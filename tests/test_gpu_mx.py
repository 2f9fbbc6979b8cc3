"""MX expert weights on the GPU, both formats (MXFP4: E2M1 codes, MXFP6: E2M3
codes): the packed layout (bit-exact against its definition in
include/dlm.h) and the grouped expert GEMM that reads it, against float64
products of the same bf16 activations and decoded weights (OCP Microscaling
v1.0: element value times the block's E8M0 scale, decoded by
oracle/numerics.py).  Model-level parity of MX experts runs in
tests/test_gpu_parity.py, tests/test_gpu_depth.py and
tests/test_gpu_fullsize.py."""
import ctypes

import numpy as np
import pytest
import torch

from oracle.numerics import mxfp4_decode, mxfp6_decode

pytestmark = pytest.mark.gpu


def _lib():
    from masked_block_diffusion_amd import abi
    return abi, abi.load_library()


FORMATS = {"mxfp4": 4, "mxfp6": 6}


def _dtype(abi, fmt):
    return {"mxfp4": abi.DLM_MXFP4, "mxfp6": abi.DLM_MXFP6}[fmt]


def _random_mx(rng, fmt, batch, N, K, zero_expert=None):
    """Random element codes [batch, N, K], E8M0 scales and the row-major code
    bytes of the format (MXFP4: element 2i in the low nibble of byte i;
    MXFP6: element 4i + j at bits 6j of the little-endian 24-bit group i)."""
    bits = FORMATS[fmt]
    codes = rng.integers(0, 1 << bits, size=(batch, N, K), dtype=np.uint8)
    scales = rng.integers(121, 130, size=(batch, N, K // 32), dtype=np.uint8)    # 2^-6 .. 2^2
    if zero_expert is not None:
        codes[zero_expert] = 0
    if bits == 4:
        packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    else:
        c = codes.astype(np.uint32).reshape(batch, N, K // 4, 4)
        g = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
        packed = np.stack([g & 255, (g >> 8) & 255, g >> 16], axis=-1).reshape(batch, N, -1).astype(np.uint8)
    return codes, packed, scales


def _decode(fmt, codes, scales):
    return (mxfp4_decode if fmt == "mxfp4" else mxfp6_decode)(codes, scales)


def _pack_reference(fmt, packed, scales):
    """The layout of include/dlm.h, written out."""
    bits = FORMATS[fmt]
    b, N, nb = packed.shape
    K = nb * 8 // bits
    rb = 128 * bits // 8
    nT, G = K // 128, (N + 15) // 16
    co = np.zeros((b, G, nT, 16, rb), dtype=np.uint8)
    so = np.full((b, G, nT, 64), 127, dtype=np.uint8)
    for n in range(N):
        for t in range(nT):
            co[:, n // 16, t, n % 16, :] = packed[:, n, rb * t:rb * t + rb]
            for j in range(4):
                so[:, n // 16, t, n % 16 + 16 * j] = scales[:, n, 4 * t + j]
    return co.reshape(-1), so.reshape(-1)


def _pack(lib, abi, fmt, packed, scales):
    b, N, nb = packed.shape
    K = nb * 8 // FORMATS[fmt]
    dt = _dtype(abi, fmt)
    nc, ns = lib.dlm_packed_mx_bytes(dt, b, N, K, 0), lib.dlm_packed_mx_bytes(dt, b, N, K, 1)
    q, e = torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda()
    dc = torch.full((nc,), 0xAB, dtype=torch.uint8, device="cuda")
    ds = torch.full((ns,), 0xCD, dtype=torch.uint8, device="cuda")
    abi.check(lib.dlm_pack_mx(dt, b, N, K, q.data_ptr(), e.data_ptr(), dc.data_ptr(), ds.data_ptr(),
                              torch.cuda.current_stream().cuda_stream), "pack_mx")
    return dc, ds


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("batch,N,K", [(3, 37, 384), (1, 16, 128), (2, 64, 2560)])
def test_pack_mx_matches_layout_definition(fmt, batch, N, K):
    abi, lib = _lib()
    rng = np.random.default_rng(batch * 1000 + N)
    _, packed, scales = _random_mx(rng, fmt, batch, N, K)
    dt, bits = _dtype(abi, fmt), FORMATS[fmt]
    assert lib.dlm_packed_mx_bytes(dt, batch, N, K, 0) == batch * ((N + 15) // 16 * 16) * K * bits // 8
    assert lib.dlm_packed_mx_bytes(dt, batch, N, K, 1) == batch * ((N + 15) // 16 * 16) * K // 32
    dc, ds = _pack(lib, abi, fmt, packed, scales)
    torch.cuda.synchronize()
    want_c, want_s = _pack_reference(fmt, packed, scales)
    assert np.array_equal(dc.cpu().numpy(), want_c)
    assert np.array_equal(ds.cpu().numpy(), want_s)


@pytest.mark.parametrize("fmt", list(FORMATS))
def test_pack_mx_rejects_bad_args(fmt):
    abi, lib = _lib()
    dt = _dtype(abi, fmt)
    q = torch.zeros(2 * 16 * 96, dtype=torch.uint8, device="cuda")
    e = torch.zeros(2 * 16 * 4, dtype=torch.uint8, device="cuda")
    d = torch.zeros(8192, dtype=torch.uint8, device="cuda")
    dp, half = d.data_ptr(), d.data_ptr() + 4096
    assert lib.dlm_packed_mx_bytes(dt, 2, 16, 100, 0) == 0
    assert lib.dlm_packed_mx_bytes(abi.DLM_BF16, 2, 16, 128, 0) == 0
    assert lib.dlm_pack_mx(abi.DLM_BF16, 2, 16, 128, q.data_ptr(), e.data_ptr(), dp, half, None) == abi.DLM_E_DTYPE
    assert lib.dlm_pack_mx(dt, 2, 16, 100, q.data_ptr(), e.data_ptr(), dp, half, None) == abi.DLM_E_SHAPE
    assert lib.dlm_pack_mx(dt, 2, 16, 128, q.data_ptr(), e.data_ptr(), q.data_ptr(), dp,
                           None) == abi.DLM_E_ARG          # output overlaps the input codes
    assert lib.dlm_pack_mx(dt, 2, 16, 128, q.data_ptr() + 8, e.data_ptr(), dp, half,
                           None) == abi.DLM_E_ARG          # misaligned codes
    assert lib.dlm_pack_mx(dt, 0, 16, 128, q.data_ptr(), e.data_ptr(), dp, half, None) == abi.DLM_E_ARG


def _mx_gemm(abi, lib, fmt, swiglu, counts, N, K, A, B, S, B2, S2, variant):
    E = len(counts)
    M = int(sum(counts))
    nws = lib.dlm_op_mx_gemm_workspace(E)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16 if swiglu else torch.float32, device="cuda")
    cnt = (ctypes.c_int32 * E)(*counts)
    abi.check(lib.dlm_op_mx_gemm(_dtype(abi, fmt), swiglu, E, cnt, N, K, A.data_ptr(), B.data_ptr(), S.data_ptr(),
                                 B2.data_ptr() if B2 is not None else None, S2.data_ptr() if S2 is not None else None,
                                 C.data_ptr(), ws.data_ptr(), nws, variant, None,
                                 torch.cuda.current_stream().cuda_stream), "mx_gemm")
    torch.cuda.synchronize()
    return C.double().cpu()


CASES = [
    # (counts per expert, N, K): empty and single-row experts, 1..4 row subtiles,
    # several m-tiles of one expert, ragged N, an odd number of 128-element
    # super-steps (a chunk of one), the full-width gate/up and down shapes
    ((0, 1, 17, 64, 130, 5), 200, 384),
    ((3,), 16, 128),
    ((40, 0, 33, 9), 768, 2560),
    ((12, 50, 7), 2560, 768),
]


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("swiglu", [0, 1])
@pytest.mark.parametrize("counts,N,K", CASES)
def test_mx_gemm_matches_fp64(fmt, swiglu, counts, N, K):
    """Every output of the grouped MX GEMM against the float64 product of the
    same bf16 activations and decoded weights.  Products are exact in fp32
    (8 significant bits times at most 4, times a power of two); the fp32 sums
    are off by at most K * 2^-24 of sum |a||w|.  SwiGLU: the bf16 store adds
    half an ulp, and the accumulation errors propagate through silu(g) * u."""
    abi, lib = _lib()
    E = len(counts)
    rng = np.random.default_rng(sum(counts) * 7 + N + K + FORMATS[fmt])
    codes, packed, scales = _random_mx(rng, fmt, E, N, K, zero_expert=0 if E > 2 else None)
    codes2, packed2, scales2 = _random_mx(rng, fmt, E, N, K)
    W = _decode(fmt, codes, scales)                       # [E, N, K] float64
    W2 = _decode(fmt, codes2, scales2)
    M = sum(counts)
    A = (torch.randn(M, K, generator=torch.Generator().manual_seed(M + K)) * 0.5).to(torch.bfloat16)
    Ad = A.double().numpy()
    B, S = _pack(lib, abi, fmt, packed, scales)
    B2, S2 = _pack(lib, abi, fmt, packed2, scales2) if swiglu else (None, None)
    got = _mx_gemm(abi, lib, fmt, swiglu, list(counts), N, K, A.cuda(), B, S, B2, S2, 0).numpy()
    r0 = 0
    for e, c in enumerate(counts):
        a = Ad[r0:r0 + c]
        ref = a @ W[e].T
        bound = (np.abs(a) @ np.abs(W[e]).T) * K * 2.0 ** -24 + 1e-30
        if not swiglu:
            assert np.all(np.abs(got[r0:r0 + c] - ref) <= bound), f"expert {e}"
        else:
            ref2 = a @ W2[e].T
            bound2 = (np.abs(a) @ np.abs(W2[e]).T) * K * 2.0 ** -24 + 1e-30
            want = ref / (1.0 + np.exp(-ref)) * ref2
            tol = np.abs(want) * 2.0 ** -8 + bound * (np.abs(ref2) + 1) + bound2 * (np.abs(ref) + 1) + 1e-6
            assert np.all(np.abs(got[r0:r0 + c] - want) <= tol), f"expert {e}"
        r0 += c


@pytest.mark.parametrize("fmt", list(FORMATS))
@pytest.mark.parametrize("variant", [1, 2, 3, 4, 5])
def test_mx_gemm_variants_identical(fmt, variant):
    """Every tile variant gives the bits of the default one: the same K order
    per output (the super-step's permuted k-steps in sequence), only the
    workgroup shape and prefetch depth change."""
    abi, lib = _lib()
    counts, N, K = (40, 0, 70, 3), 512, 640
    rng = np.random.default_rng(variant)
    _, packed, scales = _random_mx(rng, fmt, len(counts), N, K)
    _, packed2, scales2 = _random_mx(rng, fmt, len(counts), N, K)
    A = (torch.randn(sum(counts), K, generator=torch.Generator().manual_seed(3)) * 0.5).to(torch.bfloat16).cuda()
    B, S = _pack(lib, abi, fmt, packed, scales)
    B2, S2 = _pack(lib, abi, fmt, packed2, scales2)
    for swiglu in (0, 1):
        base = _mx_gemm(abi, lib, fmt, swiglu, list(counts), N, K, A, B, S, B2, S2, 0)
        other = _mx_gemm(abi, lib, fmt, swiglu, list(counts), N, K, A, B, S, B2, S2, variant)
        assert torch.equal(base, other)


def test_mx_gemm_rejects_bad_args():
    abi, lib = _lib()
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    x = torch.empty(1 << 16, dtype=torch.uint8, device="cuda")
    cnt = (ctypes.c_int32 * 2)(3, 4)
    p = x.data_ptr()

    def call(E=2, counts=cnt, N=16, K=128, variant=0, ws_bytes=4096, dtype=abi.DLM_MXFP4):
        return lib.dlm_op_mx_gemm(dtype, 0, E, counts, N, K, p, p, p, None, None, p, ws.data_ptr(), ws_bytes,
                                  variant, None, None)
    assert call(dtype=abi.DLM_BF16) == abi.DLM_E_DTYPE
    assert call(dtype=abi.DLM_MXFP6, K=96) == abi.DLM_E_SHAPE
    assert call(K=100) == abi.DLM_E_SHAPE
    assert call(E=0) == abi.DLM_E_ARG
    assert call(variant=9) == abi.DLM_E_ARG
    assert call(ws_bytes=8) == abi.DLM_E_WORKSPACE
    assert call(counts=(ctypes.c_int32 * 2)(0, 0)) == abi.DLM_E_ARG
    assert call(counts=(ctypes.c_int32 * 2)(-1, 4)) == abi.DLM_E_ARG
