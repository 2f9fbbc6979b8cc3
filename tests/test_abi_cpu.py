"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import masked_block_diffusion_amd.abi as abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dlm.h")


def _lib():
    if not os.path.exists(abi.LIB_PATH):
        pytest.skip("libdlm.so not built")
    return abi.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dlm_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(abi.EXPORTS)


def test_library_exports_every_declared_symbol():
    _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", abi.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dlm_\w+)", out))
    missing = set(header_functions()) - exported
    assert not missing, f"not exported: {sorted(missing)}"


def test_struct_sizes_match_the_c_layout():
    # 17 int/float fields; 22 pointers; 4 pointers + a pointer; seq: p, i, i, p, p, i (+pad)
    assert ctypes.sizeof(abi.dlm_config) == 17 * 4
    assert ctypes.sizeof(abi.dlm_layer_weights) == 22 * 8
    assert ctypes.sizeof(abi.dlm_weights) == 5 * 8
    assert ctypes.sizeof(abi.dlm_seq) == 8 + 4 + 4 + 8 + 8 + 8
    assert ctypes.sizeof(abi.dlm_commit_rule) == 4 + 4 + 8 + 8


def _cfg(**kw):
    c = dict(n_layers=2, d_model=128, n_q_heads=4, n_kv_heads=4, head_dim=32, vocab=512,
             mask_id=511, ffn=abi.DLM_FFN_DENSE, d_ffn=512, n_experts=0, top_k=0, d_expert=0,
             dtype=abi.DLM_F32, canvas=32, rms_eps=1e-6, rope_base=10000.0)
    c.update(kw)
    return abi.dlm_config(**c)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), abi.DLM_E_SHAPE),
    (dict(n_q_heads=6, n_kv_heads=4), abi.DLM_E_SHAPE),
    (dict(mask_id=512), abi.DLM_E_ARG),
    (dict(mask_id=-1), abi.DLM_E_ARG),
    (dict(dtype=7), abi.DLM_E_DTYPE),
    (dict(ffn=3), abi.DLM_E_ARG),
    (dict(canvas=0), abi.DLM_E_SHAPE),
    (dict(canvas=2048), abi.DLM_E_SHAPE),
    (dict(d_model=98), abi.DLM_E_SHAPE),            # 392 bytes: not a multiple of 16
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=300, top_k=8, d_expert=64), abi.DLM_E_SHAPE),
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=8, top_k=9, d_expert=64), abi.DLM_E_SHAPE),
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=64, top_k=17, d_expert=64), abi.DLM_E_SHAPE),
    (dict(n_layers=0), abi.DLM_E_SHAPE),
    # MX experts: only for bf16 MoE models, d_model and d_expert multiples of 128
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=8, top_k=2, d_expert=128, expert_dtype=abi.DLM_MXFP4), abi.DLM_E_DTYPE),
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=8, top_k=2, d_expert=64, dtype=abi.DLM_BF16,
          expert_dtype=abi.DLM_MXFP4), abi.DLM_E_SHAPE),
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=8, top_k=2, d_expert=128, dtype=abi.DLM_BF16, expert_dtype=7),
     abi.DLM_E_DTYPE),
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=8, top_k=2, d_expert=128, dtype=abi.DLM_FP8,
          expert_dtype=abi.DLM_MXFP4), abi.DLM_E_DTYPE),
    # MXFP6 experts: the same rules
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=8, top_k=2, d_expert=128, expert_dtype=abi.DLM_MXFP6), abi.DLM_E_DTYPE),
    (dict(ffn=abi.DLM_FFN_MOE, n_experts=8, top_k=2, d_expert=192, dtype=abi.DLM_BF16,
          expert_dtype=abi.DLM_MXFP6), abi.DLM_E_SHAPE),
])
def test_create_rejects_bad_config(kw, status):
    lib = _lib()
    c = _cfg(**kw)
    h = ctypes.c_void_p()
    w = abi.dlm_weights()
    assert lib.dlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == status
    assert h.value is None
    assert lib.dlm_last_error().decode()


def test_create_rejects_missing_weights():
    lib = _lib()
    c = _cfg()
    h = ctypes.c_void_p()
    assert lib.dlm_create(ctypes.byref(c), None, ctypes.byref(h)) == abi.DLM_E_ARG
    w = abi.dlm_weights()                           # all NULL
    assert lib.dlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.byref(h)) == abi.DLM_E_ARG
    # fp8 without scales
    layers = (abi.dlm_layer_weights * 2)()
    for L in layers:
        for f, _ in abi.dlm_layer_weights._fields_:
            if not f.endswith("_s") and f not in ("w_router", "we_gate", "we_up", "we_down"):
                setattr(L, f, 0x1000)
    w = abi.dlm_weights(embed=0x1000, final_norm=0x1000, lm_head=0x1000, lm_head_s=0x1000,
                        layers=ctypes.cast(layers, ctypes.POINTER(abi.dlm_layer_weights)))
    c8 = _cfg(dtype=abi.DLM_FP8)
    assert lib.dlm_create(ctypes.byref(c8), ctypes.byref(w), ctypes.byref(h)) == abi.DLM_E_DTYPE
    assert "scale" in lib.dlm_last_error().decode()


def test_calls_on_null_model_fail_cleanly():
    lib = _lib()
    assert lib.dlm_workspace_bytes(None, 32, 96) == 0
    seq = abi.dlm_seq()
    assert lib.dlm_prefill(None, ctypes.byref(seq), None, 4, None, 0, None) == abi.DLM_E_ARG
    arr = (ctypes.POINTER(abi.dlm_seq) * 1)(ctypes.pointer(seq))
    assert lib.dlm_denoise_step(None, arr, 1, None, None, None, None, 0, None) == abi.DLM_E_ARG
    assert lib.dlm_append_canvas(None, arr, 1, None, 0, None) == abi.DLM_E_ARG
    rule = abi.dlm_commit_rule()
    assert lib.dlm_commit(None, arr, 1, None, None, ctypes.byref(rule), 0, None, None, None) == abi.DLM_E_ARG
    assert lib.dlm_check_device_status(None, None, None) == abi.DLM_E_ARG
    assert lib.dlm_timing_enable(None, 1) == abi.DLM_E_ARG
    assert lib.dlm_debug_router(None, None, None, 0) == abi.DLM_E_ARG
    lib.dlm_destroy(None)                           # no-op


def test_kernel_names():
    lib = _lib()
    names = [lib.dlm_kernel_name(i).decode() for i in range(abi.DLM_K_COUNT)]
    assert all(names) and len(set(names)) == abi.DLM_K_COUNT
    assert lib.dlm_kernel_name(abi.DLM_K_COUNT).decode() == ""
    assert names[abi.DLM_K_LM_HEAD] == "lm_head"


def test_pack_weight_validates_on_the_host():
    """dlm_packed_weight_bytes is host arithmetic (16-row padding); bad
    dtype / shape / pointers are refused before any HIP call."""
    lib = _lib()
    assert lib.dlm_packed_weight_bytes(abi.DLM_BF16, 3, 40, 64) == 3 * 48 * 64 * 2
    assert lib.dlm_packed_weight_bytes(abi.DLM_FP8, 1, 16, 128) == 16 * 128
    assert lib.dlm_packed_weight_bytes(abi.DLM_F32, 1, 1, 32) == 16 * 32 * 4
    assert lib.dlm_packed_weight_bytes(abi.DLM_BF16, 1, 16, 100) == 0        # K * 2 not a multiple of 128
    assert lib.dlm_packed_weight_bytes(7, 1, 16, 64) == 0
    assert lib.dlm_packed_weight_bytes(abi.DLM_BF16, 0, 16, 64) == 0
    assert lib.dlm_pack_weight(abi.DLM_BF16, 1, 16, 64, None, None, None) == abi.DLM_E_ARG
    assert lib.dlm_pack_weight(abi.DLM_BF16, 1, 16, 100, 0x1000, 0x100000, None) == abi.DLM_E_SHAPE
    assert lib.dlm_pack_weight(9, 1, 16, 64, 0x1000, 0x100000, None) == abi.DLM_E_DTYPE
    assert lib.dlm_pack_weight(abi.DLM_BF16, 1, 16, 64, 0x1000, 0x1000 + 100, None) == abi.DLM_E_ARG   # overlap


def test_op_route_validates_on_the_host():
    """The routing test hook checks every expert id (a host array) and its
    workspace before any HIP call; ids outside [0, E) never reach a kernel."""
    import numpy as np
    lib = _lib()
    assert lib.dlm_op_route_workspace(0, 8) == 0 and lib.dlm_op_route_workspace(10, 257) == 0
    need = lib.dlm_op_route_workspace(100, 16)
    assert need > 0
    ids = np.zeros(100, dtype=np.int32)
    p = ids.ctypes.data
    fake = 0x1000
    assert lib.dlm_op_route(None, 100, 16, 64, fake, fake, fake, fake, fake, need, None) == abi.DLM_E_ARG
    assert lib.dlm_op_route(p, 100, 0, 64, fake, fake, fake, fake, fake, need, None) == abi.DLM_E_ARG
    assert lib.dlm_op_route(p, 100, 16, 0, fake, fake, fake, fake, fake, need, None) == abi.DLM_E_ARG
    ids[57] = 16
    assert lib.dlm_op_route(p, 100, 16, 64, fake, fake, fake, fake, fake, need, None) == abi.DLM_E_ARG
    assert b"ids[57]" in lib.dlm_last_error()
    ids[57] = -1
    assert lib.dlm_op_route(p, 100, 16, 64, fake, fake, fake, fake, fake, need, None) == abi.DLM_E_ARG
    ids[57] = 3
    assert lib.dlm_op_route(p, 100, 16, 64, fake, fake, fake, fake, fake, need - 1, None) == abi.DLM_E_WORKSPACE


def test_op_router_topk_validates_on_the_host():
    lib = _lib()
    f = 0x1000
    assert lib.dlm_op_router_topk(None, 4, 8, 2, f, f, None) == abi.DLM_E_ARG
    assert lib.dlm_op_router_topk(f, 0, 8, 2, f, f, None) == abi.DLM_E_ARG
    assert lib.dlm_op_router_topk(f, 4, 257, 2, f, f, None) == abi.DLM_E_ARG
    assert lib.dlm_op_router_topk(f, 4, 8, 9, f, f, None) == abi.DLM_E_ARG
    assert lib.dlm_op_router_topk(f, 4, 32, 17, f, f, None) == abi.DLM_E_ARG


def test_mx_pack_and_gemm_validate_on_the_host():
    """Packed MX sizes are host arithmetic (16-row padding; codes K * bits / 8
    and scales K / 32 bytes per row, bits 4 for MXFP4 and 6 for MXFP6); bad
    dtypes, shapes and pointers are refused before any HIP call."""
    lib = _lib()
    f4, f6 = abi.DLM_MXFP4, abi.DLM_MXFP6
    assert lib.dlm_packed_mx_bytes(f4, 3, 40, 256, 0) == 3 * 48 * 128
    assert lib.dlm_packed_mx_bytes(f6, 3, 40, 256, 0) == 3 * 48 * 192
    assert lib.dlm_packed_mx_bytes(f4, 3, 40, 256, 1) == 3 * 48 * 8
    assert lib.dlm_packed_mx_bytes(f6, 3, 40, 256, 1) == 3 * 48 * 8
    assert lib.dlm_packed_mx_bytes(abi.DLM_BF16, 1, 16, 128, 0) == 0       # not an MX format
    assert lib.dlm_packed_mx_bytes(f6, 1, 16, 192, 0) == 0                  # K not a multiple of 128
    assert lib.dlm_packed_mx_bytes(f4, 0, 16, 128, 0) == 0
    assert lib.dlm_pack_mx(abi.DLM_FP8, 1, 16, 128, 0x1000, 0x2000, 0x10000, 0x20000, None) == abi.DLM_E_DTYPE
    for f in (f4, f6):
        assert lib.dlm_pack_mx(f, 1, 16, 128, None, None, None, None, None) == abi.DLM_E_ARG
        assert lib.dlm_pack_mx(f, 1, 16, 192, 0x1000, 0x2000, 0x10000, 0x20000, None) == abi.DLM_E_SHAPE
        assert lib.dlm_pack_mx(f, 1, 16, 128, 0x1008, 0x2000, 0x10000, 0x20000, None) == abi.DLM_E_ARG  # misaligned
        assert lib.dlm_pack_mx(f, 1, 16, 128, 0x1000, 0x2000, 0x1000, 0x20000, None) == abi.DLM_E_ARG   # overlap
    # MXFP6 codes of 16 rows x 128 elements are 1536 bytes: an output 1024
    # bytes past them overlaps, one 2048 bytes past does not
    assert lib.dlm_pack_mx(f6, 1, 16, 128, 0x10000, 0x2000, 0x10400, 0x20000, None) == abi.DLM_E_ARG
    cnt = (ctypes.c_int32 * 2)(3, 4)
    assert lib.dlm_op_mx_gemm_workspace(0) == 0
    assert lib.dlm_op_mx_gemm(abi.DLM_BF16, 0, 2, cnt, 16, 128, 0x1000, 0x1000, 0x1000, None, None, 0x1000,
                              0x1000, 4096, 0, None, None) == abi.DLM_E_DTYPE
    assert lib.dlm_op_mx_gemm(f4, 0, 2, cnt, 16, 128, None, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 4096, 0,
                              None, None) == abi.DLM_E_ARG
    assert lib.dlm_op_mx_gemm(f6, 0, 2, cnt, 16, 96, 0x1000, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 4096, 0,
                              None, None) == abi.DLM_E_SHAPE
    assert lib.dlm_op_mx_gemm(f4, 1, 2, cnt, 16, 128, 0x1000, 0x1000, 0x1000, None, None, 0x1000, 0x1000, 4096, 0,
                              None, None) == abi.DLM_E_ARG                   # SwiGLU without B2 / S2
