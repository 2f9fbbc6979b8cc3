"""Workload shapes for block-diffusion denoising.

This module holds only dimensions, schedules' parameters and seeds: no arithmetic
of the method. Both the CPU oracle and the HIP path read these tables.

The five full-size workloads follow the pages' statement of the problem: a
causally prefilled prefix, a 256-token all-[MASK] canvas denoised over a fixed or
adaptive number of steps, and the canvas appended to the KV cache when full
(rahulsharmavishwakarma.github.io "Diffusion LLMs: what changes...", section 4.2,
"Block decoding" and "Few steps"; b4rtaz.github.io "Diffusion LLMs are not a good
fit for distributed inference", canvas paragraph).  The layer shapes are not on
the pages; they are the dimensions of the workload definitions this project is
measured on.  The "mini" variants shrink every dimension so the oracle finishes
in seconds while still spanning several kernel tiles and ragged tails.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class ModelConfig:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    vocab: int
    mask_id: int
    ffn: str                 # "dense" or "moe"
    d_ffn: int               # dense SwiGLU inner dim; for "moe" the shared expert's inner dim
    n_experts: int = 0
    top_k: int = 0
    d_expert: int = 0
    dtype: str = "bf16"      # "f32", "bf16" or "fp8": weights and GEMM operands
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    init_std: float = 0.02
    router_std: Optional[float] = None   # None -> d_model ** -0.5
    lm_head_std: Optional[float] = None  # None -> init_std; larger values give peaked confidences
    expert_dtype: Optional[str] = None   # MoE experts' storage when it differs from dtype: "mxfp4", "mxfp6"

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def qkv_dim(self) -> int:
        return self.q_dim + 2 * self.kv_dim

    @property
    def router_sigma(self) -> float:
        return self.router_std if self.router_std is not None else self.d_model ** -0.5

    def n_params(self) -> dict:
        d, L = self.d_model, self.n_layers
        attn = d * self.qkv_dim + self.q_dim * d
        dense = 3 * d * self.d_ffn
        experts = 3 * d * self.d_expert * self.n_experts if self.ffn == "moe" else 0
        router = d * self.n_experts if self.ffn == "moe" else 0
        active_experts = 3 * d * self.d_expert * self.top_k if self.ffn == "moe" else 0
        return {
            "embed": self.vocab * d,
            "lm_head": self.vocab * d,
            "per_layer_total": attn + dense + experts + router,
            "total": L * (attn + dense + experts + router) + 2 * self.vocab * d,
            "active_compute": L * (attn + dense + active_experts + router) + self.vocab * d,
        }


@dataclass(frozen=True)
class RunConfig:
    name: str
    model: ModelConfig
    canvas: int                       # C: tokens per canvas
    n_requests: int                   # R: independent sequences denoised together
    prefix_len: Tuple[int, int]       # (lo, hi) inclusive; lo == hi for a fixed length
    n_canvases: int
    rule: str                         # "topk" (fixed schedule) or "threshold"
    n_steps: int                      # steps per canvas (maximum for "threshold")
    threshold: float = 0.5
    page_size: int = 64               # KV page size in tokens (paged layout)
    seed: int = 0
    edit_threshold: float = 0.0       # token editing (T2T): > 0 rewrites earlier tokens (0: off)

    @property
    def max_prefix(self) -> int:
        return self.prefix_len[1]

    def capacity(self) -> int:
        """Tokens of KV cache one request needs: prefix + all canvases."""
        return self.max_prefix + self.n_canvases * self.canvas


# ---- models -----------------------------------------------------------------

TINY_DENSE_F32 = ModelConfig(
    name="tiny-dense-f32", n_layers=2, d_model=128, n_q_heads=4, n_kv_heads=4,
    head_dim=32, vocab=512, mask_id=511, ffn="dense", d_ffn=512, dtype="f32")

DENSE_BF16 = ModelConfig(
    name="dense-16L-2048-bf16", n_layers=16, d_model=2048, n_q_heads=16, n_kv_heads=4,
    head_dim=128, vocab=32768, mask_id=32767, ffn="dense", d_ffn=8192, dtype="bf16")

MOE_BF16 = ModelConfig(
    name="moe-26b-a3b-bf16", n_layers=32, d_model=2560, n_q_heads=20, n_kv_heads=4,
    head_dim=128, vocab=262144, mask_id=262143, ffn="moe", d_ffn=2048,
    n_experts=128, top_k=8, d_expert=768, dtype="bf16")

MOE_FP8 = replace(MOE_BF16, name="moe-26b-a3b-fp8", dtype="fp8")

# the same model with its routed experts' weights in MXFP4 (4.25 bits per weight)
MOE_MXFP4 = replace(MOE_BF16, name="moe-26b-a3b-mxfp4", expert_dtype="mxfp4")

# ... and in MXFP6, E2M3 elements (6.25 bits per weight)
MOE_MXFP6 = replace(MOE_BF16, name="moe-26b-a3b-mxfp6", expert_dtype="mxfp6")

# Reduced models for oracle-speed parity: same structure, small dims, ragged
# vocab (not a multiple of any tile) so tails are exercised.
DENSE_BF16_MINI = ModelConfig(
    name="dense-mini-bf16", n_layers=2, d_model=512, n_q_heads=4, n_kv_heads=1,
    head_dim=128, vocab=4000, mask_id=3999, ffn="dense", d_ffn=1024, dtype="bf16")

MOE_BF16_MINI = ModelConfig(
    name="moe-mini-bf16", n_layers=2, d_model=512, n_q_heads=4, n_kv_heads=1,
    head_dim=128, vocab=4000, mask_id=3999, ffn="moe", d_ffn=256,
    n_experts=16, top_k=4, d_expert=128, dtype="bf16")

MOE_FP8_MINI = replace(MOE_BF16_MINI, name="moe-mini-fp8", dtype="fp8")

MOE_MXFP4_MINI = replace(MOE_BF16_MINI, name="moe-mini-mxfp4", expert_dtype="mxfp4")
MOE_MXFP6_MINI = replace(MOE_BF16_MINI, name="moe-mini-mxfp6", expert_dtype="mxfp6")

DENSE_FP8_MINI = replace(DENSE_BF16_MINI, name="dense-mini-fp8", dtype="fp8")

# the bf16 attention kernel's smaller head sizes (4 waves per workgroup)
DENSE_BF16_MINI_DH64 = replace(DENSE_BF16_MINI, name="dense-mini-dh64-bf16", n_q_heads=8, n_kv_heads=2, head_dim=64)
DENSE_BF16_MINI_DH32 = replace(DENSE_BF16_MINI, name="dense-mini-dh32-bf16", n_q_heads=16, n_kv_heads=4, head_dim=32)


# ---- runs -------------------------------------------------------------------

RUNS = {
    # 1: tiny dense fp32, 64-token prefix, 32-token canvas, 8 steps x 4 commits
    "tiny": RunConfig("tiny", TINY_DENSE_F32, canvas=32, n_requests=1,
                      prefix_len=(64, 64), n_canvases=1, rule="topk", n_steps=8),
    # 2: dense bf16, 1024 prefix, 256 canvas, 16 steps x 16, then append
    "dense": RunConfig("dense", DENSE_BF16, canvas=256, n_requests=1,
                       prefix_len=(1024, 1024), n_canvases=1, rule="topk", n_steps=16),
    # 3: 26B-class MoE bf16, 4096 prefix, 4 canvases x 12 steps
    "moe": RunConfig("moe", MOE_BF16, canvas=256, n_requests=1,
                     prefix_len=(4096, 4096), n_canvases=4, rule="topk", n_steps=12),
    # 4: same model in fp8, threshold 0.5, <= 48 steps, one canvas
    "moe-fp8": RunConfig("moe-fp8", MOE_FP8, canvas=256, n_requests=1,
                         prefix_len=(4096, 4096), n_canvases=1, rule="threshold",
                         n_steps=48, threshold=0.5),
    # 3 with MXFP4 routed experts
    "moe-mxfp4": RunConfig("moe-mxfp4", MOE_MXFP4, canvas=256, n_requests=1,
                           prefix_len=(4096, 4096), n_canvases=4, rule="topk", n_steps=12),
    # 3 with MXFP6 routed experts
    "moe-mxfp6": RunConfig("moe-mxfp6", MOE_MXFP6, canvas=256, n_requests=1,
                           prefix_len=(4096, 4096), n_canvases=4, rule="topk", n_steps=12),
    # 5: 32 independent requests, prefixes U[512, 4096], paged KV
    "moe-batch32": RunConfig("moe-batch32", MOE_BF16, canvas=256, n_requests=32,
                             prefix_len=(512, 4096), n_canvases=1, rule="topk",
                             n_steps=12),
    # reduced variants (parity at oracle speed)
    "dense-mini": RunConfig("dense-mini", DENSE_BF16_MINI, canvas=256, n_requests=1,
                            prefix_len=(100, 100), n_canvases=2, rule="topk", n_steps=16),
    "dense-mini-ragged": RunConfig("dense-mini-ragged", DENSE_BF16_MINI, canvas=40,
                                   n_requests=1, prefix_len=(37, 37), n_canvases=2,
                                   rule="topk", n_steps=7),
    "moe-mini": RunConfig("moe-mini", MOE_BF16_MINI, canvas=64, n_requests=1,
                          prefix_len=(100, 100), n_canvases=2, rule="topk", n_steps=12),
    "moe-mini-fp8": RunConfig("moe-mini-fp8", MOE_FP8_MINI, canvas=64, n_requests=1,
                              prefix_len=(100, 100), n_canvases=1, rule="threshold",
                              n_steps=48, threshold=0.5),
    "dense-mini-fp8": RunConfig("dense-mini-fp8", DENSE_FP8_MINI, canvas=64, n_requests=1,
                                prefix_len=(70, 70), n_canvases=1, rule="threshold",
                                n_steps=48, threshold=0.5),
    "dense-mini-dh64": RunConfig("dense-mini-dh64", DENSE_BF16_MINI_DH64, canvas=48, n_requests=1,
                                 prefix_len=(77, 77), n_canvases=2, rule="topk", n_steps=6),
    "dense-mini-dh32": RunConfig("dense-mini-dh32", DENSE_BF16_MINI_DH32, canvas=48, n_requests=2,
                                 prefix_len=(30, 140), n_canvases=1, rule="topk", n_steps=6),
    "moe-mini-mxfp4": RunConfig("moe-mini-mxfp4", MOE_MXFP4_MINI, canvas=64, n_requests=1,
                                prefix_len=(100, 100), n_canvases=2, rule="topk", n_steps=12),
    "moe-mini-mxfp4-batch": RunConfig("moe-mini-mxfp4-batch", MOE_MXFP4_MINI, canvas=64, n_requests=4,
                                      prefix_len=(20, 150), n_canvases=1, rule="topk", n_steps=12),
    "moe-mini-mxfp6": RunConfig("moe-mini-mxfp6", MOE_MXFP6_MINI, canvas=64, n_requests=1,
                                prefix_len=(100, 100), n_canvases=2, rule="topk", n_steps=12),
    "moe-mini-mxfp6-batch": RunConfig("moe-mini-mxfp6-batch", MOE_MXFP6_MINI, canvas=64, n_requests=4,
                                      prefix_len=(20, 150), n_canvases=1, rule="topk", n_steps=12),
    "moe-mini-batch": RunConfig("moe-mini-batch", MOE_BF16_MINI, canvas=64, n_requests=4,
                                prefix_len=(20, 150), n_canvases=1, rule="topk",
                                n_steps=12),
    # a long prompt on the reduced MoE: its prefill routes 8400 assignments over
    # 16 experts (>= 512 per expert), the compute-bound expert tiles' regime
    "moe-mini-longprompt": RunConfig("moe-mini-longprompt", MOE_BF16_MINI, canvas=64, n_requests=1,
                                     prefix_len=(2100, 2100), n_canvases=1, rule="topk", n_steps=12),
    # token editing on the tiny model: the threshold sits inside the spread of its
    # confidences (~1/V), so some earlier tokens are rewritten and some are not
    "tiny-t2t": RunConfig("tiny-t2t", TINY_DENSE_F32, canvas=32, n_requests=1,
                          prefix_len=(64, 64), n_canvases=2, rule="topk", n_steps=8,
                          edit_threshold=0.0040),
    # the dense model with editing on wherever the prediction moved (timing of the
    # edit pass; random-init confidences are ~1/V)
    "dense-t2t": RunConfig("dense-t2t", DENSE_BF16, canvas=256, n_requests=1,
                           prefix_len=(1024, 1024), n_canvases=1, rule="topk", n_steps=16,
                           edit_threshold=1e-6),
}


def get_run(name: str) -> RunConfig:
    try:
        return RUNS[name]
    except KeyError:
        raise KeyError(f"unknown run {name!r}; known: {sorted(RUNS)}") from None
