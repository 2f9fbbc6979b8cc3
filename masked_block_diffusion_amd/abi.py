"""ctypes mirror of include/dlm.h and the loader of libdlm.so.

Argument marshalling only: every struct here has the field order and types of
its C counterpart, and every function is the C entry point of the same name.
The library is loaded after torch so that it binds to the HIP runtime torch
already loaded (both carry the soname libamdhip64.so.7): one runtime, so torch
streams and device pointers are valid inside the library.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_size_t, c_void_p

import torch  # noqa: F401  (must be loaded before libdlm.so; see module doc)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdlm.so")

DLM_OK = 0
DLM_E_ARG = -1
DLM_E_SHAPE = -2
DLM_E_DTYPE = -3
DLM_E_CAPACITY = -4
DLM_E_STATE = -5
DLM_E_WORKSPACE = -6
DLM_E_HIP = -7
DLM_E_DEVICE = -8
DLM_E_UNSUPPORTED = -9

DLM_DEVERR_TOKEN_RANGE = 1
DLM_DEVERR_MASK_APPEND = 2
DLM_MAX_SEQS = 64
DLM_STATIC_SCRATCH_BYTES = 128 << 20

DLM_F32, DLM_BF16, DLM_FP8, DLM_MXFP4, DLM_MXFP6 = 0, 1, 2, 3, 4
DLM_FFN_DENSE, DLM_FFN_MOE = 0, 1
DLM_COMMIT_TOPK, DLM_COMMIT_THRESHOLD = 0, 1

KERNEL_IDS = [
    "DLM_K_EMBED", "DLM_K_NORM", "DLM_K_GEMM_QKV", "DLM_K_ROPE_KV", "DLM_K_ATTN",
    "DLM_K_ATTN_MERGE", "DLM_K_GEMM_O", "DLM_K_GEMM_GATE_UP", "DLM_K_GEMM_DOWN",
    "DLM_K_QUANT", "DLM_K_ROUTER", "DLM_K_TOPK", "DLM_K_PERMUTE", "DLM_K_EXPERT_GATE_UP",
    "DLM_K_EXPERT_DOWN", "DLM_K_COMBINE", "DLM_K_LM_HEAD", "DLM_K_LM_MERGE", "DLM_K_COMMIT",
    "DLM_K_SPLITK_EPILOGUE",
]
for _i, _n in enumerate(KERNEL_IDS):
    globals()[_n] = _i
DLM_K_COUNT = len(KERNEL_IDS)

# Every symbol include/dlm.h declares.
EXPORTS = [
    "dlm_create", "dlm_destroy", "dlm_workspace_bytes", "dlm_prefill", "dlm_denoise_step",
    "dlm_commit", "dlm_append_canvas", "dlm_check_device_status", "dlm_last_error",
    "dlm_timing_enable", "dlm_timing_read", "dlm_kernel_name", "dlm_debug_router",
    "dlm_op_quant_rows", "dlm_op_gemm", "dlm_op_gemm_workspace", "dlm_packed_weight_bytes", "dlm_pack_weight",
    "dlm_op_route", "dlm_op_route_workspace", "dlm_op_router_topk", "dlm_denoise_step_noalloc",
    "dlm_packed_mx_bytes", "dlm_pack_mx", "dlm_op_mx_gemm", "dlm_op_mx_gemm_workspace",
]
DLM_GEMM_B_TILED = 0x100


class dlm_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32), ("head_dim", c_int32), ("vocab", c_int32),
        ("mask_id", c_int32), ("ffn", c_int32), ("d_ffn", c_int32), ("n_experts", c_int32),
        ("top_k", c_int32), ("d_expert", c_int32), ("dtype", c_int32), ("canvas", c_int32),
        ("rms_eps", c_float), ("rope_base", c_float), ("expert_dtype", c_int32),
    ]


class dlm_layer_weights(ctypes.Structure):
    _fields_ = [
        ("attn_norm", c_void_p), ("ffn_norm", c_void_p),
        ("wqkv", c_void_p), ("wqkv_s", c_void_p),
        ("wo", c_void_p), ("wo_s", c_void_p),
        ("w_gate", c_void_p), ("w_gate_s", c_void_p),
        ("w_up", c_void_p), ("w_up_s", c_void_p),
        ("w_down", c_void_p), ("w_down_s", c_void_p),
        ("w_router", c_void_p),
        ("we_gate", c_void_p), ("we_gate_s", c_void_p),
        ("we_up", c_void_p), ("we_up_s", c_void_p),
        ("we_down", c_void_p), ("we_down_s", c_void_p),
        ("we_gate_e8", c_void_p), ("we_up_e8", c_void_p), ("we_down_e8", c_void_p),
    ]


class dlm_weights(ctypes.Structure):
    _fields_ = [
        ("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
        ("lm_head_s", c_void_p), ("layers", POINTER(dlm_layer_weights)),
    ]


class dlm_seq(ctypes.Structure):
    _fields_ = [
        ("kv", c_void_p), ("capacity", c_int32), ("T", c_int32), ("canvas", c_void_p),
        ("page_table", c_void_p), ("page_size", c_int32),
    ]


class dlm_commit_rule(ctypes.Structure):
    _fields_ = [
        ("kind", c_int32), ("n_steps", c_int32), ("k_per_step", POINTER(c_int32)),
        ("threshold", c_float), ("edit_threshold", c_float),
    ]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads libdlm.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m masked_block_diffusion_amd.build`")
    lib = ctypes.CDLL(path)
    P = c_void_p
    sig = {
        "dlm_create": (c_int32, [POINTER(dlm_config), POINTER(dlm_weights), POINTER(c_void_p)]),
        "dlm_destroy": (None, [P]),
        "dlm_workspace_bytes": (c_size_t, [P, c_int32, c_int32]),
        "dlm_prefill": (c_int32, [P, POINTER(dlm_seq), P, c_int32, P, c_size_t, P]),
        "dlm_denoise_step": (c_int32, [P, POINTER(POINTER(dlm_seq)), c_int32, P, P, P, P, c_size_t, P]),
        "dlm_denoise_step_noalloc": (c_int32, [P, POINTER(POINTER(dlm_seq)), c_int32, P, P, P, P]),
        "dlm_commit": (c_int32, [P, POINTER(POINTER(dlm_seq)), c_int32, P, P, POINTER(dlm_commit_rule),
                                 c_int32, P, P, P]),
        "dlm_append_canvas": (c_int32, [P, POINTER(POINTER(dlm_seq)), c_int32, P, c_size_t, P]),
        "dlm_check_device_status": (c_int32, [P, P, POINTER(c_int32)]),
        "dlm_last_error": (c_char_p, []),
        "dlm_timing_enable": (c_int32, [P, c_int32]),
        "dlm_timing_read": (c_int32, [P, POINTER(c_float), POINTER(c_int32)]),
        "dlm_kernel_name": (c_char_p, [c_int32]),
        "dlm_debug_router": (c_int32, [P, P, P, ctypes.c_int64]),
        "dlm_op_quant_rows": (c_int32, [P, c_int32, c_int32, P, P, P]),
        "dlm_op_gemm": (c_int32, [c_int32, c_int32, c_int32, c_int32, c_int32, P, P, P, P, P, P, P, P,
                                  c_size_t, c_int32, c_int32, POINTER(c_float), P]),
        "dlm_op_gemm_workspace": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
        "dlm_packed_weight_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
        "dlm_pack_weight": (c_int32, [c_int32, c_int32, c_int32, c_int32, P, P, P]),
        "dlm_op_route": (c_int32, [P, c_int32, c_int32, c_int32, P, P, P, P, P, c_size_t, P]),
        "dlm_op_route_workspace": (c_size_t, [c_int32, c_int32]),
        "dlm_op_router_topk": (c_int32, [P, c_int32, c_int32, c_int32, P, P, P]),
        "dlm_packed_mx_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32]),
        "dlm_pack_mx": (c_int32, [c_int32, c_int32, c_int32, c_int32, P, P, P, P, P]),
        "dlm_op_mx_gemm": (c_int32, [c_int32, c_int32, c_int32, POINTER(c_int32), c_int32, c_int32, P, P, P, P, P,
                                     P, P, c_size_t, c_int32, POINTER(c_float), P]),
        "dlm_op_mx_gemm_workspace": (c_size_t, [c_int32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


class DLMError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where} failed with status {status}: {detail}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != DLM_OK:
        raise DLMError(status, where, load_library().dlm_last_error().decode())
