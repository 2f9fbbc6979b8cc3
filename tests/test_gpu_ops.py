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


@pytest.mark.parametrize("pad8", [False, True], ids=["odd-width", "width-multiple-of-8"])
def test_quant_rows_exhaustive_bf16(pad8):
    """Both quantiser paths: rows of odd width (element loop) and rows padded
    with zeros to a multiple of 8 (16-byte chunks kept in registers); zero
    padding changes no row maximum and quantises to code 0."""
    import ctypes
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    bits = _bf16_rows()
    if pad8:
        bits = np.pad(bits, ((0, 0), (0, (-bits.shape[1]) % 8)))
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


def _bf16_tensor(shape, g):
    return (torch.randn(*shape, generator=g) * 0.5).to(torch.bfloat16)


@pytest.mark.parametrize("variant,splits", [(v, 0) for v in range(13)] + [(3, 2), (2, 4), (1, 3), (0, 5), (9, 2), (9, 4), (10, 3)])
@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (37, 200, 1536), (256, 512, 2048), (300, 136, 256)])
def test_gemm_variants_match_fp64(variant, splits, M, N, K):
    """Every tile variant and split factor of the dense GEMM, ragged M / N,
    against a float64 product of the same bf16 values (fp32 accumulation:
    relative error bounded by K * 2^-24 of sum |a||b|)."""
    import ctypes
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    g = torch.Generator().manual_seed(M * 1000 + N + K)
    A, B, B2 = _bf16_tensor((M, K), g), _bf16_tensor((N, K), g), _bf16_tensor((N, K), g)
    ref = A.double() @ B.double().T
    ref2 = A.double() @ B2.double().T
    bound = (A.double().abs() @ B.double().abs().T) * K * 2.0 ** -24 + 1e-30
    bound2 = (A.double().abs() @ B2.double().abs().T) * K * 2.0 ** -24 + 1e-30
    st = torch.cuda.current_stream().cuda_stream
    for swiglu in (0, 1):
        nws = lib.dlm_op_gemm_workspace(abi.DLM_BF16, swiglu, M, N, K, variant, splits)
        ws = torch.empty(max(nws, 4), dtype=torch.uint8, device="cuda")
        C = torch.empty((M, N), dtype=torch.float32 if not swiglu else torch.bfloat16, device="cuda")
        Ad, Bd, B2d = A.cuda(), B.cuda(), B2.cuda()
        abi.check(lib.dlm_op_gemm(abi.DLM_BF16, swiglu, M, N, K, Ad.data_ptr(), Bd.data_ptr(), B2d.data_ptr(),
                                  None, None, None, C.data_ptr(), ws.data_ptr(), ws.numel(), variant, splits,
                                  None, st), "gemm")
        torch.cuda.synchronize()
        got = C.double().cpu()
        if not swiglu:
            assert torch.all((got - ref).abs() <= bound), f"max excess {((got - ref).abs() - bound).max()}"
        else:
            want = torch.nn.functional.silu(ref) * ref2
            # the bf16 store rounds: half an ulp of the result, plus the propagated accumulation error
            tol = want.abs() * 2.0 ** -8 + bound * (ref2.abs() + 1) + bound2 * (ref.abs() + 1) + 1e-6
            assert torch.all((got - want).abs() <= tol), f"max excess {((got - want).abs() - tol).max()}"


def test_gemm_wide_tile_matches_fp64():
    """A prefill-sized single-weight GEMM that takes the wide 128 x 256 tile
    (17 x 16 tiles, ragged in both M and N) against a float64 product of the
    same bf16 values (fp32 accumulation: K * 2^-24 of sum |a||b|)."""
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    M, N, K = 2100, 4000, 256
    g = torch.Generator().manual_seed(11)
    A, B = _bf16_tensor((M, K), g), _bf16_tensor((N, K), g)
    ref = A.double() @ B.double().T
    bound = (A.double().abs() @ B.double().abs().T) * K * 2.0 ** -24 + 1e-30
    st = torch.cuda.current_stream().cuda_stream
    nws = lib.dlm_op_gemm_workspace(abi.DLM_BF16, 0, M, N, K, 0, 0)
    ws = torch.empty(max(nws, 4), dtype=torch.uint8, device="cuda")
    C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    Ad, Bd = A.cuda(), B.cuda()
    abi.check(lib.dlm_op_gemm(abi.DLM_BF16, 0, M, N, K, Ad.data_ptr(), Bd.data_ptr(), None, None, None, None,
                              C.data_ptr(), ws.data_ptr(), ws.numel(), 0, 0, None, st), "gemm")
    torch.cuda.synchronize()
    got = C.double().cpu()
    assert torch.all((got - ref).abs() <= bound), f"max excess {((got - ref).abs() - bound).max()}"


def test_gemm_f32_matches_fp64():
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    g = torch.Generator().manual_seed(7)
    M, N, K = 32, 520, 128
    A, B = torch.randn(M, K, generator=g), torch.randn(N, K, generator=g)
    ref = A.double() @ B.double().T
    bound = (A.double().abs() @ B.double().abs().T) * K * 2.0 ** -22
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    nws = lib.dlm_op_gemm_workspace(abi.DLM_F32, 0, M, N, K, 0, 0)
    ws = torch.empty(max(nws, 4), dtype=torch.uint8, device="cuda")
    Ad, Bd = A.cuda(), B.cuda()          # keep both alive while the kernel runs
    abi.check(lib.dlm_op_gemm(abi.DLM_F32, 0, M, N, K, Ad.data_ptr(), Bd.data_ptr(), None, None, None, None,
                              C.data_ptr(), ws.data_ptr(), ws.numel(), 0, 0, None, st), "gemm")
    torch.cuda.synchronize()
    assert torch.all((C.double().cpu() - ref).abs() <= bound)


@pytest.mark.parametrize("M,N,K,splits", [(256, 320, 512, 0), (64, 128, 2560, 0), (37, 200, 768, 2),
                                          (300, 64, 128, 0)])
def test_gemm_fp8_matches_fp64(M, N, K, splits):
    """E4M3 codes covering every finite value (subnormals, both zeros) with
    per-row / per-column scales, against the oracle's decoding in float64.
    Products of two E4M3 values are exact in fp32; the sum is fp32."""
    from masked_block_diffusion_amd import abi
    from oracle.numerics import e4m3_decode
    lib = abi.load_library()
    rng = np.random.default_rng(M + N + K)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    A = rng.choice(finite, size=(M, K)).astype(np.uint8)
    B = rng.choice(finite, size=(N, K)).astype(np.uint8)
    B2 = rng.choice(finite, size=(N, K)).astype(np.uint8)
    sa = rng.uniform(0.5, 2.0, M).astype(np.float32)
    sb = rng.uniform(0.5, 2.0, N).astype(np.float32)
    sb2 = rng.uniform(0.5, 2.0, N).astype(np.float32)
    Ad, Bd, B2d = e4m3_decode(A), e4m3_decode(B), e4m3_decode(B2)
    raw = Ad @ Bd.T
    ref = raw * sa[:, None].astype(np.float64) * sb[None, :].astype(np.float64)
    bound = (np.abs(Ad) @ np.abs(Bd).T) * K * 2.0 ** -24 * sa[:, None] * sb[None, :] + np.abs(ref) * 2.0 ** -22
    t = {k: torch.from_numpy(v).cuda() for k, v in dict(A=A, B=B, B2=B2, sa=sa, sb=sb, sb2=sb2).items()}
    st = torch.cuda.current_stream().cuda_stream
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nws = lib.dlm_op_gemm_workspace(abi.DLM_FP8, 0, M, N, K, 0, splits)
    ws = torch.empty(max(nws, 4), dtype=torch.uint8, device="cuda")
    abi.check(lib.dlm_op_gemm(abi.DLM_FP8, 0, M, N, K, t["A"].data_ptr(), t["B"].data_ptr(), t["B2"].data_ptr(),
                              t["sa"].data_ptr(), t["sb"].data_ptr(), t["sb2"].data_ptr(), C.data_ptr(),
                              ws.data_ptr(), ws.numel(), 0, splits, None, st), "gemm fp8")
    torch.cuda.synchronize()
    got = C.cpu().numpy().astype(np.float64)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (f"{bad.sum()} of {bad.size} differ; worst rel "
                           f"{np.max(np.abs(got - ref) / (np.abs(ref) + 1e-30)):.3g}; "
                           f"e.g. got {got[bad][:3]} want {ref[bad][:3]}")


def test_gemm_fp8_small_integers_exact():
    """E4M3 codes of small integers (1..16, both signs) with unit scales: every
    partial sum is an integer below 2^24, so any summation order is exact."""
    from masked_block_diffusion_amd import abi
    from oracle.numerics import e4m3_decode, e4m3_encode
    lib = abi.load_library()
    rng = np.random.default_rng(5)
    M, N, K = 300, 136, 512
    vals = np.array([v for v in range(-16, 17) if v != 0 and abs(e4m3_decode(e4m3_encode(v))) == abs(v)], float)
    A = e4m3_encode(rng.choice(vals, size=(M, K)))
    B = e4m3_encode(rng.choice(vals, size=(N, K)))
    ref = e4m3_decode(A) @ e4m3_decode(B).T
    t = {k: torch.from_numpy(v).cuda() for k, v in dict(A=A, B=B).items()}
    ones_m = torch.ones(M, dtype=torch.float32, device="cuda")
    ones_n = torch.ones(N, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for variant_m in (M, 64, 256):                 # the three tile classes (prefill / small / canvas)
        mm = min(M, variant_m)
        C = torch.empty((mm, N), dtype=torch.float32, device="cuda")
        nws = lib.dlm_op_gemm_workspace(abi.DLM_FP8, 0, mm, N, K, 0, 0)
        ws = torch.empty(max(nws, 4), dtype=torch.uint8, device="cuda")
        abi.check(lib.dlm_op_gemm(abi.DLM_FP8, 0, mm, N, K, t["A"].data_ptr(), t["B"].data_ptr(), None,
                                  ones_m.data_ptr(), ones_n.data_ptr(), None, C.data_ptr(), ws.data_ptr(),
                                  ws.numel(), 0, 0, None, st), "gemm fp8")
        torch.cuda.synchronize()
        got = C.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref[:mm]), f"M={mm}: {np.sum(got != ref[:mm])} differ"


def test_paged_cache_validation():
    """Page tables need 64-token pages and a capacity of whole pages; a page
    size without a table is an argument error."""
    import synth
    from masked_block_diffusion_amd import DLM, KVPool, abi
    run = synth.get_run("tiny")
    gm = DLM(run.model, {k: v.cuda() for k, v in synth.make_weights(run.model).items()}, canvas=run.canvas)
    pool = KVPool(gm, 4)
    seq = gm.new_seq(128, pool)
    ids = synth.make_inputs(run)[0].cuda()
    ws = gm.workspace(len(ids), 128)
    for page_size, cap, status in ((16, 128, abi.DLM_E_UNSUPPORTED), (64, 96, abi.DLM_E_SHAPE)):
        seq.raw.page_size, seq.raw.capacity = page_size, cap
        with pytest.raises(abi.DLMError) as e:
            gm.dlm_prefill(seq, ids, ws)
        assert e.value.status == status
    seq.raw.page_size, seq.raw.capacity = 64, 128
    plain = gm.new_seq(128)
    plain.raw.page_size = 64
    with pytest.raises(abi.DLMError) as e:
        gm.dlm_prefill(plain, ids, ws)
    assert e.value.status == abi.DLM_E_ARG
    gm.dlm_prefill(seq, ids, ws)
    torch.cuda.synchronize()
    assert seq.T == len(ids)
    gm.close()


def _pack_reference(w_bytes: np.ndarray) -> np.ndarray:
    """The tiled layout from its definition in include/dlm.h, on the CPU:
    w_bytes uint8 [batch, N, K*eb] -> blocks of 16 rows x 128 bytes, block
    (n // 16, kt) at ((n // 16) * nkt + kt) * 2048, rows padded with zeros."""
    b, N, rb = w_bytes.shape
    Np = (N + 15) // 16 * 16
    pad = np.zeros((b, Np, rb), dtype=np.uint8)
    pad[:, :N] = w_bytes
    nkt = rb // 128
    out = np.zeros(b * Np * rb, dtype=np.uint8)
    for m in range(b):
        for n in range(Np):
            for kt in range(nkt):
                off = m * Np * rb + ((n // 16) * nkt + kt) * 2048 + (n % 16) * 128
                out[off:off + 128] = pad[m, n, kt * 128:(kt + 1) * 128]
    return out


@pytest.mark.parametrize("dtype,batch,N,K", [("f32", 1, 40, 64), ("bf16", 3, 64, 128), ("bf16", 2, 37, 320),
                                             ("fp8", 4, 24, 256), ("fp8", 1, 16, 128)])
def test_pack_weight_matches_layout_definition(dtype, batch, N, K):
    """dlm_pack_weight writes exactly the documented byte layout (bit-exact),
    ragged N padded with zero rows, expert batches one after another."""
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    code = {"f32": abi.DLM_F32, "bf16": abi.DLM_BF16, "fp8": abi.DLM_FP8}[dtype]
    eb = {"f32": 4, "bf16": 2, "fp8": 1}[dtype]
    rng = np.random.default_rng(batch * 100 + N)
    src = rng.integers(0, 256, size=(batch, N, K * eb), dtype=np.uint8)
    nbytes = lib.dlm_packed_weight_bytes(code, batch, N, K)
    assert nbytes == batch * ((N + 15) // 16 * 16) * K * eb
    s = torch.from_numpy(src.copy()).cuda()
    d = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    abi.check(lib.dlm_pack_weight(code, batch, N, K, s.data_ptr(), d.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream), "pack")
    torch.cuda.synchronize()
    assert np.array_equal(d.cpu().numpy(), _pack_reference(src))
    # overlapping buffers are refused before anything is enqueued
    assert lib.dlm_pack_weight(code, batch, N, K, s.data_ptr(), s.data_ptr(), None) == abi.DLM_E_ARG


@pytest.mark.parametrize("variant,splits", [(0, 0), (2, 2), (9, 0), (3, 3), (7, 0)])
@pytest.mark.parametrize("M,N,K", [(37, 200, 1536), (256, 512, 2048), (5, 72, 256)])
def test_gemm_tiled_weights_bit_identical(variant, splits, M, N, K):
    """The GEMM reading tiled weights (the layout the model uses) gives the
    same bits as reading the row-major matrix: only addresses change."""
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    g = torch.Generator().manual_seed(M + N + K)
    A, B, B2 = _bf16_tensor((M, K), g).cuda(), _bf16_tensor((N, K), g).cuda(), _bf16_tensor((N, K), g).cuda()
    st = torch.cuda.current_stream().cuda_stream

    def tiled(w):
        d = torch.empty(lib.dlm_packed_weight_bytes(abi.DLM_BF16, 1, N, K), dtype=torch.uint8, device="cuda")
        abi.check(lib.dlm_pack_weight(abi.DLM_BF16, 1, N, K, w.data_ptr(), d.data_ptr(), st), "pack")
        return d
    Bt, B2t = tiled(B), tiled(B2)
    for swiglu in (0, 1):
        outs = []
        for flag, (b, b2) in ((0, (B, B2)), (abi.DLM_GEMM_B_TILED, (Bt, B2t))):
            v = variant | flag
            nws = lib.dlm_op_gemm_workspace(abi.DLM_BF16, swiglu, M, N, K, v, splits)
            ws = torch.empty(max(nws, 4), dtype=torch.uint8, device="cuda")
            C = torch.empty((M, N), dtype=torch.float32 if not swiglu else torch.bfloat16, device="cuda")
            abi.check(lib.dlm_op_gemm(abi.DLM_BF16, swiglu, M, N, K, A.data_ptr(), b.data_ptr(), b2.data_ptr(),
                                      None, None, None, C.data_ptr(), ws.data_ptr(), ws.numel(), v, splits,
                                      None, st), "gemm")
            outs.append(C)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("n,E,bm,dist", [(1, 1, 64, "uniform"), (64, 256, 64, "uniform"), (2048, 128, 64, "uniform"),
                                         (2048, 128, 64, "one"), (4096, 256, 32, "skewed"), (4096, 128, 128, "uniform"),
                                         (4097, 128, 64, "uniform"), (4097, 256, 64, "skewed"), (1000, 7, 32, "uniform"),
                                         (65536, 128, 128, "uniform"), (32768, 128, 64, "one")])
def test_route_sort_bit_exact(n, E, bm, dist):
    """The expert sort of the MoE layer (one-workgroup path up to 4096
    assignments, three kernels beyond) against a stable sort on the CPU:
    offsets, m-tile starts, order by (expert, assignment) and its inverse, bit
    for bit, including 256 experts, a single expert and the path boundary."""
    import numpy as np
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    rng = np.random.default_rng(n * 7 + E)
    if dist == "uniform":
        ids = rng.integers(0, E, n)
    elif dist == "one":
        ids = np.full(n, E - 1)
    else:                                             # a few hot experts
        ids = np.minimum(rng.geometric(0.05, n) - 1, E - 1)
    ids = ids.astype(np.int32)
    counts = np.bincount(ids, minlength=E)
    offs_ref = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    tiles_ref = np.concatenate([[0], np.cumsum((counts + bm - 1) // bm)]).astype(np.int32)
    sorted_ref = np.argsort(ids, kind="stable").astype(np.int32)
    inv_ref = np.empty(n, dtype=np.int32)
    inv_ref[sorted_ref] = np.arange(n, dtype=np.int32)
    dev = "cuda"
    offs = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    tiles = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    srt = torch.full((n,), -7, dtype=torch.int32, device=dev)
    inv = torch.full((n,), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(lib.dlm_op_route_workspace(n, E), dtype=torch.uint8, device=dev)
    abi.check(lib.dlm_op_route(ids.ctypes.data, n, E, bm, offs.data_ptr(), tiles.data_ptr(), srt.data_ptr(),
                               inv.data_ptr(), ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream),
              "route")
    torch.cuda.synchronize()
    assert np.array_equal(offs.cpu().numpy(), offs_ref)
    assert np.array_equal(tiles.cpu().numpy(), tiles_ref)
    assert np.array_equal(srt.cpu().numpy(), sorted_ref)
    assert np.array_equal(inv.cpu().numpy(), inv_ref)


@pytest.mark.parametrize("rows,E,k", [(1, 1, 1), (257, 128, 8), (64, 256, 16), (33, 16, 4), (5, 7, 7)])
def test_router_topk_ties_and_weights(rows, E, k):
    """The router's top-k on logits with many exact ties (small integers):
    experts in decreasing logit order with ties to the lower id, exactly as a
    stable sort on the CPU; weights = softmax renormalised over the chosen k
    (fp32 against float64, relative 1e-6)."""
    import numpy as np
    from masked_block_diffusion_amd import abi
    lib = abi.load_library()
    rng = np.random.default_rng(rows * 3 + E)
    logits = rng.integers(-3, 4, size=(rows, E)).astype(np.float32) * 0.5
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(logits.astype(np.float64), order, axis=1)
    p = np.exp(sel - logits.max(axis=1, keepdims=True))
    w_ref = p / p.sum(axis=1, keepdims=True)
    d = torch.from_numpy(logits).cuda()
    ids = torch.full((rows, k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((rows, k), dtype=torch.float32, device="cuda")
    abi.check(lib.dlm_op_router_topk(d.data_ptr(), rows, E, k, ids.data_ptr(), w.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream), "router_topk")
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), order.astype(np.int32))
    assert np.allclose(w.cpu().numpy(), w_ref, rtol=1e-6, atol=0)


@pytest.mark.parametrize("C", [32, 1000])
def test_commit_ties_bit_exact(C):
    """dlm_commit on hand-built confidences drawn from three values (ties
    everywhere), some positions already committed, three requests: the
    top-k rule (ties -> lower position) and the threshold rule (inclusive at
    the threshold, the single most confident when none reaches it, every
    masked position at the last step) against the oracle's commit functions,
    canvases and counts bit for bit."""
    import numpy as np
    import synth
    from masked_block_diffusion_amd import DLM, Rule
    from oracle import sampler as osampler
    run = synth.get_run("tiny")
    cfg = run.model
    w = synth.make_weights(cfg, seed=run.seed)
    gm = DLM(cfg, {k: v.to("cuda:0") for k, v in w.items()}, canvas=C, device="cuda:0")
    R, mask = 3, cfg.mask_id
    rng = np.random.default_rng(C)
    seqs = [gm.new_seq(C + 64) for _ in range(R)]
    # (rule, steps, step): top-k of C // steps (+1) per step, all of C at one
    # step; threshold 0.5 at a first step, a middle step and the last (forced)
    cases = [("topk", 1, 0), ("topk", 3, 2), ("topk", 7, 0), ("threshold", 3, 0), ("threshold", 3, 1),
             ("threshold", 3, 2)]
    for rule_kind, n_steps, step in cases:
        canv = np.where(rng.random((R, C)) < 0.7, mask, rng.integers(0, mask, (R, C))).astype(np.int32)
        canv[1, :] = mask                                       # request 1 fully masked
        conf = rng.choice(np.float32([0.25, 0.5, 0.75]), size=(R, C)).astype(np.float32)
        if rule_kind == "threshold":
            conf[2] = np.float32(0.25)                          # request 2: nothing reaches 0.5
        pred = rng.integers(0, mask, (R, C)).astype(np.int32)
        if rule_kind == "topk":
            k = osampler.topk_schedule(C, n_steps)[step]
            rule = Rule.topk(C, n_steps)
        else:
            rule = Rule.threshold(n_steps, 0.5)
        for i, s in enumerate(seqs):
            s.canvas.copy_(torch.from_numpy(canv[i]))
        conf_d = torch.from_numpy(conf.reshape(-1)).cuda()
        pred_d = torch.from_numpy(pred.reshape(-1)).cuda()
        ncom = torch.full((R,), -1, dtype=torch.int32, device="cuda")
        nmask = torch.full((R,), -1, dtype=torch.int32, device="cuda")
        gm.dlm_commit(seqs, conf_d, pred_d, rule, step, ncom, nmask)
        torch.cuda.synchronize()
        for i, s in enumerate(seqs):
            if rule_kind == "topk":
                want, chosen = osampler.commit_topk(canv[i], conf[i], pred[i], mask, k)
            else:
                want, chosen = osampler.commit_threshold(canv[i], conf[i], pred[i], mask, 0.5, step, n_steps)
            got = s.canvas.cpu().numpy()
            assert np.array_equal(got, want), (rule_kind, step, i)
            assert int(ncom[i]) == len(chosen)
            assert int(nmask[i]) == int((want == mask).sum())
    gm.close()


@pytest.mark.parametrize("name", ["tiny", "dense-mini"])
def test_lm_head_argmax_ties(name):
    """The LM head's fused reduction on exact ties: the head is zero except
    three identical rows (two ids in one vocabulary tile, one in another) and
    the [MASK] row at ten times that vector.  Every canvas row then ties --
    among the three (where h.v > 0) or among all the zero rows -- and the
    prediction must be the lowest tied id, never [MASK], with confidence
    1 / sum exp(l - max) over the non-[MASK] logits the kernel exposes."""
    import numpy as np
    import synth
    from masked_block_diffusion_amd import DLM
    run = synth.get_run(name)
    cfg, C = run.model, run.canvas
    w = synth.make_weights(cfg, seed=run.seed)
    lm = w["lm_head"]
    g = torch.Generator().manual_seed(5)
    v = (torch.randn(cfg.d_model, generator=g) * 0.05).to(lm.dtype)
    lm.zero_()
    tied = [70, 71, 300]
    for t in tied:
        lm[t] = v
    lm[cfg.mask_id] = (v.float() * 10).to(lm.dtype)
    if cfg.dtype == "fp8":
        pytest.skip("fp8 heads are quantised codes")
    gm = DLM(cfg, {k: x.to("cuda:0") for k, x in w.items()}, canvas=C, device="cuda:0")
    ids = synth.make_inputs(run)[0].to("cuda:0")
    seq = gm.new_seq(run.capacity())
    ws = gm.workspace(max(C, len(ids)), run.capacity())
    gm.dlm_prefill(seq, ids, ws)
    conf = torch.empty(C, dtype=torch.float32, device="cuda:0")
    pred = torch.empty(C, dtype=torch.int32, device="cuda:0")
    logits = torch.empty(C * cfg.vocab, dtype=torch.float32, device="cuda:0")
    gm.dlm_denoise_step([seq], conf, pred, ws, logits)
    torch.cuda.synchronize()
    L = logits.view(C, cfg.vocab).double().cpu().numpy()
    keep = np.arange(cfg.vocab) != cfg.mask_id
    got_pred, got_conf = pred.cpu().numpy(), conf.cpu().numpy()
    kinds = set()
    for r in range(C):
        lr = np.where(keep, L[r], -np.inf)
        mx = lr.max()
        assert L[r, tied[0]] == L[r, tied[1]] == L[r, tied[2]]          # the ties are exact in the kernel
        want = int(np.nonzero(lr == mx)[0][0])
        kinds.add(want)
        assert got_pred[r] == want, (r, got_pred[r], want)
        assert got_pred[r] != cfg.mask_id
        z = np.exp(lr[keep] - mx).sum()
        assert abs(got_conf[r] - 1.0 / z) <= 1e-5 / z
    assert kinds <= {0, tied[0]}
    gm.close()
