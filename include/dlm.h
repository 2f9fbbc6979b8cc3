/*
 * dlm.h -- C ABI of the block-diffusion denoising library (libdlm.so, gfx950).
 *
 * The library runs the hot path of a block-diffusion language model:
 *
 *   1. dlm_prefill        causal forward over a prompt; writes every layer's
 *                         post-RoPE K and V into the request's KV cache.
 *   2. dlm_denoise_step   one bidirectional forward over the canvas (all
 *                         canvas positions see each other and the whole
 *                         cached prefix), the LM head, and per position the
 *                         greedy prediction and its confidence.
 *   3. dlm_commit         turns the most confident still-masked positions into
 *                         their predicted tokens.
 *   4. dlm_append_canvas  forward over the finished canvas with the denoising
 *                         mask; its K/V become part of the cache (T += C).
 *
 * Where these come from ("What changes" = rahulsharmavishwakarma.github.io,
 * "Diffusion LLMs: what changes when you stop generating one token at a time"):
 *   - reverse process: start all-[MASK], predict masked positions, commit the
 *     most confident ones, repeat until nothing is masked (What changes, sec. 2);
 *   - bidirectional attention inside the block and several commits per pass
 *     (What changes, sec. 2, properties 1 and 2);
 *   - autoregressive across blocks, diffusion within a block, with KV caching
 *     (What changes, sec. 4.1);
 *   - a 256-token canvas, causal prefill, bidirectional denoising, finished
 *     canvases appended to the KV cache, up to 48 steps (What changes,
 *     sec. 4.2 "Block decoding" and "Few steps");
 *   - committing only positions above a confidence threshold (What changes,
 *     sec. 5, "Quality vs steps").
 * The pages give no layer internals; the model is a pre-RMSNorm transformer
 * with rotary embeddings, grouped-query attention, a SwiGLU FFN (dense, or a
 * softmax-top-k mixture of SwiGLU experts plus an ungated shared expert) and an
 * untied LM head.  [MASK] is excluded from the prediction; confidence is the
 * maximum softmax probability over the remaining vocabulary; ties in the
 * prediction go to the lower token id and ties in confidence rank to the lower
 * position.
 *
 * Conventions for every entry point:
 *   - Memory: the caller allocates and frees all device memory (weights, KV
 *     caches, canvases, outputs, workspace).  Pointers marked "device" must be
 *     device memory of the current HIP device; "host" pointers are read before
 *     the call returns.  The library never frees caller memory.  It owns only
 *     its host handle, one 4-byte device error word per model and, for MoE
 *     models, one HIP stream (default priority) with two events.
 *   - Streams: all GPU work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream) -- for MoE models each layer's shared expert runs on the
 *     model's own stream, forked from `stream` by an event and joined back into
 *     it before its result is used, so all work still starts after earlier work
 *     on `stream` and finishes before later work on it.  No entry point
 *     synchronises except dlm_check_device_status and dlm_timing_read.  One
 *     model handle serves one stream at a time.
 *   - Errors: arguments are validated on the host before anything is enqueued;
 *     on failure the call returns a negative dlm_status, enqueues nothing and
 *     changes no state, and dlm_last_error() describes the failure.  Faults only
 *     the device can see (a token id outside the vocabulary, a masked position
 *     in a canvas being appended) set the model's device error word, which
 *     dlm_check_device_status reports.  Nothing throws across the ABI.
 *   - No entry point allocates device memory after dlm_create, and none issues
 *     hipMemset, so a caller may capture dlm_denoise_step / dlm_commit into a
 *     HIP graph.
 *   - Host state: dlm_prefill and dlm_append_canvas advance dlm_seq.T on the
 *     host when they return DLM_OK.
 */
#ifndef DLM_H
#define DLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t dlm_status;
#define DLM_OK            0
#define DLM_E_ARG        -1   /* null pointer, bad enum, bad count */
#define DLM_E_SHAPE      -2   /* dimensions the kernels cannot take */
#define DLM_E_DTYPE      -3   /* dtype / weight set mismatch */
#define DLM_E_CAPACITY   -4   /* KV cache too small for the call */
#define DLM_E_STATE      -5   /* call not valid in the current state */
#define DLM_E_WORKSPACE  -6   /* workspace null or smaller than dlm_workspace_bytes */
#define DLM_E_HIP        -7   /* a HIP runtime call failed */
#define DLM_E_DEVICE     -8   /* the device error word is set */
#define DLM_E_UNSUPPORTED -9  /* valid request the library does not implement */

/* Bits of the device error word. */
#define DLM_DEVERR_TOKEN_RANGE   1   /* an input id was < 0 or >= vocab */
#define DLM_DEVERR_MASK_APPEND   2   /* dlm_append_canvas saw a [MASK] */

#define DLM_MAX_SEQS 64              /* requests per denoise/commit/append call */

/* DLM_MXFP4, DLM_MXFP6: storage of the routed experts' weights only
 * (dlm_config.expert_dtype). */
typedef enum { DLM_F32 = 0, DLM_BF16 = 1, DLM_FP8 = 2, DLM_MXFP4 = 3, DLM_MXFP6 = 4 } dlm_dtype;
typedef enum { DLM_FFN_DENSE = 0, DLM_FFN_MOE = 1 } dlm_ffn_kind;

/* Model shape.  Constraints checked by dlm_create: head_dim in {32, 64, 128};
 * n_q_heads a multiple of n_kv_heads; (n_q_heads + n_kv_heads) * head_dim
 * <= 8192; d_model, d_ffn, d_expert multiples of 32
 * (f32) / 64 (bf16) / 128 (fp8) elements; top_k <= n_experts <= 256,
 * top_k <= 16; 0 <= mask_id < vocab; canvas in [1, 1024]; d_model <= 4096. */
typedef struct {
    int32_t n_layers;
    int32_t d_model;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t vocab;
    int32_t mask_id;
    int32_t ffn;        /* dlm_ffn_kind */
    int32_t d_ffn;      /* dense FFN inner dim; for MoE the shared expert's inner dim */
    int32_t n_experts;  /* MoE only */
    int32_t top_k;      /* MoE only */
    int32_t d_expert;   /* MoE only: inner dim of each expert */
    int32_t dtype;      /* dlm_dtype: storage of weights and GEMM operands */
    int32_t canvas;     /* C: tokens per canvas */
    float   rms_eps;
    float   rope_base;
    /* Storage of the routed experts' weights (MoE only; ignored for dense
     * models): equal to dtype, or with a DLM_BF16 model one of the OCP
     * Microscaling (MX) v1.0 formats, elements in blocks of 32 along K sharing
     * an E8M0 scale: DLM_MXFP4 (E2M1 elements, 4.25 bits per weight -- the
     * 4-bit expert weights of DiffusionGemma 4x, "Deployment and Tooling", in
     * the chip's own 4-bit format) or DLM_MXFP6 (E2M3 elements, 6.25 bits per
     * weight).  The experts then compute with the decoded weights (element
     * value times block scale, exact in bf16) on the bf16 activations, fp32
     * sums; the rest of the model is bf16.  MX experts need d_model and
     * d_expert multiples of 128.  E_DTYPE for any other value. */
    int32_t expert_dtype;
} dlm_config;

/* Per-layer weights, all device pointers.  Shapes are [out, in] (a GEMM computes
 * y = x W^T).  Element type: fp32 for DLM_F32, bf16 for DLM_BF16, OCP E4M3FN
 * codes (uint8) for DLM_FP8 projections.  "_s" pointers are the fp8 per-output-
 * channel fp32 scales (W = code * s[out]); NULL for other dtypes.
 * Layout: the projections (wqkv, wo, w_gate, w_up, w_down, we_gate, we_up,
 * we_down and lm_head) are in the tiled layout dlm_pack_weight writes from the
 * row-major matrix (per expert for we_*); w_router and embed are row-major.
 *   wqkv   [(Hq + 2 Hkv) * dh, d]  rows: Q heads, then K heads, then V heads
 *   wo     [d, Hq * dh]
 *   w_gate, w_up [F, d]; w_down [d, F]     F = d_ffn (dense FFN or shared expert)
 *   w_router [E, d]        bf16 (fp32 for DLM_F32) -- also for DLM_FP8 models
 *   we_gate, we_up [E, De, d]; we_down [E, d, De]
 *   attn_norm, ffn_norm [d] fp32 RMSNorm gains.                                  */
typedef struct {
    const float* attn_norm;
    const float* ffn_norm;
    const void*  wqkv;    const float* wqkv_s;
    const void*  wo;      const float* wo_s;
    const void*  w_gate;  const float* w_gate_s;
    const void*  w_up;    const float* w_up_s;
    const void*  w_down;  const float* w_down_s;
    const void*  w_router;
    const void*  we_gate; const float* we_gate_s;
    const void*  we_up;   const float* we_up_s;
    const void*  we_down; const float* we_down_s;
    /* MX experts (expert_dtype DLM_MXFP4 / DLM_MXFP6): we_gate / we_up /
     * we_down hold the packed element codes and these the packed E8M0 scales,
     * both in the layout dlm_pack_mx writes; NULL otherwise. */
    const uint8_t* we_gate_e8;
    const uint8_t* we_up_e8;
    const uint8_t* we_down_e8;
} dlm_layer_weights;

/* embed [V, d]: fp32 (DLM_F32) or bf16.  lm_head [V, d] untied, projection
 * dtype.  final_norm [d] fp32.  layers: HOST array of n_layers entries, copied
 * by dlm_create (the device tensors it points to must outlive the model). */
typedef struct {
    const void*  embed;
    const float* final_norm;
    const void*  lm_head;  const float* lm_head_s;
    const dlm_layer_weights* layers;
} dlm_weights;

/* Tiled weight layout.  Layout only -- the values are the row-major projection
 * matrices of the transformer described above, rearranged so that a GEMM's
 * K stage over 16 consecutive output rows is one contiguous 2 KB run (weights
 * stream from HBM in whole DRAM pages rather than one 128-byte line per row).
 * For a [N, K] matrix of eb-byte elements (eb = 4, 2, 1 for DLM_F32, DLM_BF16,
 * DLM_FP8), nkt = K * eb / 128: the 128 bytes of row n holding k-bytes
 * [128 kt, 128 kt + 128) sit at byte ((n / 16) * nkt + kt) * 2048 + (n % 16) * 128.
 * N is padded to a multiple of 16 with zero rows; `batch` matrices (the experts
 * of a layer) follow one another.
 * dlm_packed_weight_bytes: bytes of the packed output (0 on invalid arguments).
 * dlm_pack_weight: src device [batch, N, K] row-major, dst device (caller-
 * allocated, dlm_packed_weight_bytes long, not overlapping src); enqueued on
 * `stream`.  E_DTYPE for an unknown dtype, E_ARG for null or overlapping
 * pointers or batch / N / K < 1, E_SHAPE unless K * eb is a multiple of 128. */
size_t dlm_packed_weight_bytes(int32_t dtype, int32_t batch, int32_t N, int32_t K);
dlm_status dlm_pack_weight(int32_t dtype, int32_t batch, int32_t N, int32_t K, const void* src, void* dst,
                           void* stream);

/* MX weight layout (DLM_MXFP4: 4-bit E2M1 codes, DLM_MXFP6: 6-bit E2M3
 * codes).  Layout only: the codes and scales of OCP MX v1.0 matrices,
 * rearranged so that one wave's loads fetch 128 consecutive K elements of 16
 * rows (16 x RB bytes, RB = 128 * bits / 8 = 64 or 96) and one byte per lane
 * their 64 scales.  For a [N, K] matrix (K a multiple of 128, nT = K / 128; N
 * padded to a multiple of 16 with zero codes and scale code 127):
 *   codes:  the RB bytes of row n holding elements [128 t, 128 t + 128) sit at
 *           byte ((n / 16) * nT + t) * 16 RB + (n % 16) * RB, unchanged from
 *           the row-major codes (MXFP4: two per byte, the even element in the
 *           low nibble; MXFP6: four per 3 bytes, element 4i + j at bits 6j ..
 *           6j + 5 of the little-endian 24-bit group i);
 *   scales: the scale of row n, elements [128 t + 32 j, 128 t + 32 j + 32) sits
 *           at byte ((n / 16) * nT + t) * 64 + (n % 16) + 16 j.
 * `batch` matrices follow one another in each.
 * dlm_packed_mx_bytes: bytes of the packed codes (scales = 0) or scales
 * (scales = 1); 0 on invalid arguments.
 * dlm_pack_mx: codes device uint8 [batch, N, K * bits / 8], scales device uint8
 * [batch, N, K / 32] (E8M0 codes, one per 32 elements of a row), both
 * row-major, 16-byte aligned -> dst_codes, dst_scales (device, caller-
 * allocated, dlm_packed_mx_bytes long, overlapping no input); enqueued on
 * `stream`.  E_DTYPE unless dtype is DLM_MXFP4 or DLM_MXFP6; E_ARG for null,
 * misaligned or overlapping pointers or batch / N / K < 1; E_SHAPE unless
 * K % 128 == 0. */
size_t dlm_packed_mx_bytes(int32_t dtype, int32_t batch, int32_t N, int32_t K, int32_t scales);
dlm_status dlm_pack_mx(int32_t dtype, int32_t batch, int32_t N, int32_t K, const void* codes, const void* scales,
                       void* dst_codes, void* dst_scales, void* stream);

/* One request.  Host struct of non-owning device pointers.
 *   kv: KV cache, bf16 (fp32 for DLM_F32 models).
 *     Contiguous (page_table NULL): per layer and KV head a key block then a
 *       value block: [n_layers][2][n_kv_heads][capacity * head_dim], the key
 *       block [capacity][head_dim] (row t: the post-RoPE key of absolute
 *       position t), the value block stored transposed, [head_dim][capacity]
 *       (column t: the value of position t), so attention reads consecutive
 *       positions of one value dimension.
 *     Paged (page_table set): kv is the base of a pool of 64-token pages;
 *       position t lives in page page_table[t / 64] at slot t % 64.  A page
 *       holds all layers and heads of its tokens, [n_layers][2][n_kv_heads]
 *       [64 * head_dim], keys [64][head_dim] and transposed values
 *       [head_dim][64]; page p starts p * n_layers * 2 * n_kv_heads * 64 *
 *       head_dim elements after kv.  Requests may share a pool; the pages of
 *       one request must be distinct and not used by another request in the
 *       same call.
 *     Slots not yet written may hold anything; they are never used.
 *   capacity: tokens the cache holds; a multiple of 8 (E_SHAPE otherwise), so
 *       every transposed value row is 16-byte aligned; paged: a multiple of
 *       64, the table then has capacity / 64 entries.
 *   T: tokens cached so far (prefix plus appended canvases).
 *   canvas: device int32[C], the block being denoised ([MASK] = mask_id).
 *   page_table: device int32[capacity / 64] page indices into the pool, or
 *       NULL; page_size: 64 with a page table (E_UNSUPPORTED otherwise), 0
 *       without one (E_ARG otherwise). */
typedef struct {
    void*          kv;
    int32_t        capacity;
    int32_t        T;
    int32_t*       canvas;
    const int32_t* page_table;
    int32_t        page_size;
} dlm_seq;

/* Commit rule (What changes, sec. 2 and sec. 5).
 *   DLM_COMMIT_TOPK: at step s commit the k_per_step[s] most confident masked
 *     positions (all of them if fewer remain).
 *   DLM_COMMIT_THRESHOLD: commit every masked position with confidence >=
 *     threshold; if there is none, the single most confident one; at step
 *     n_steps - 1, every masked position.
 * k_per_step: HOST array of n_steps entries (TOPK only).
 * edit_threshold: token editing (T2T; What changes, the LLaDA2.1 item: the
 *   model may revise tokens it already wrote; the pages give no rule, this is
 *   its plainest form).  When > 0, every position that held a token before the
 *   step, whose prediction differs from it and whose confidence is >=
 *   edit_threshold, is rewritten with the prediction.  0 turns editing off
 *   (mask -> token only).  Edits never touch or write mask_id, so the masked
 *   counts follow the commit rule alone. */
typedef enum { DLM_COMMIT_TOPK = 0, DLM_COMMIT_THRESHOLD = 1 } dlm_commit_kind;
typedef struct {
    int32_t        kind;
    int32_t        n_steps;
    const int32_t* k_per_step;
    float          threshold;
    float          edit_threshold;
} dlm_commit_rule;

typedef struct dlm_model dlm_model;

/* Creates a model handle over caller-owned device weights on the current HIP
 * device.  Validates the config and that every pointer the config needs is
 * non-NULL.  Allocates the 4-byte device error word (zeroed).  */
dlm_status dlm_create(const dlm_config* cfg, const dlm_weights* weights, dlm_model** out);

/* Frees the handle and its error word.  NULL is a no-op. */
void dlm_destroy(dlm_model* model);

/* Bytes of device workspace a call needs when it processes up to `max_rows`
 * token rows in one forward (R * C for denoise/append, n for prefill) and
 * attends to up to `max_kv_tokens` keys per request.  0 on invalid input. */
size_t dlm_workspace_bytes(const dlm_model* model, int32_t max_rows, int32_t max_kv_tokens);

/* Causal forward over ids (device int32[n]) at positions [T, T + n) of `seq`;
 * K/V of every layer are written to cache slots [T, T + n); then seq->T += n.
 * No LM head.  E_CAPACITY if T + n > capacity. */
dlm_status dlm_prefill(dlm_model* model, dlm_seq* seq, const int32_t* ids, int32_t n,
                       void* ws, size_t ws_bytes, void* stream);

/* One denoising pass over the canvases of n_seqs requests.  Request r's canvas
 * sits at positions [T_r, T_r + C); its queries attend to cache slots [0, T_r)
 * and to all C canvas keys (no mask inside the canvas).  The canvas K/V are
 * written to slots [T_r, T_r + C) as scratch; T does not change.  Those K/V
 * are bit-identical to what dlm_append_canvas writes for the same canvas (the
 * same forward under the same block mask), so a caller whose canvas already
 * holds final tokens may advance seq->T by C instead of appending -- what
 * autoregressive decoding with C = 1 does (the canvas holds the newest token;
 * the pass's prediction is the next one).
 *   conf [n_seqs, C] fp32 (device, out): max softmax probability over the
 *        vocabulary without [MASK];
 *   pred [n_seqs, C] int32 (device, out): lowest-id argmax over the same set;
 *   logits [n_seqs, C, V] fp32 (device, out, nullable): raw logits, for tests.
 * E_CAPACITY if T_r + C > capacity for any request. */
dlm_status dlm_denoise_step(dlm_model* model, dlm_seq* const* seqs, int32_t n_seqs,
                            float* conf, int32_t* pred, float* logits,
                            void* ws, size_t ws_bytes, void* stream);

/* Applies the commit rule at step `step` (0-based) to each request's canvas,
 * in place: positions that hold mask_id are written per the rule (and, with
 * rule->edit_threshold > 0, earlier tokens per the editing rule), always with
 * their prediction (never with mask_id).  Ranking: higher confidence first,
 * equal confidence -> lower position first.
 *   n_committed [n_seqs] int32 (device, out, nullable): positions written
 *               (commits plus edits);
 *   n_masked    [n_seqs] int32 (device, out, nullable): positions still masked.
 * E_ARG if step is outside [0, rule->n_steps) or edit_threshold is negative or
 * not finite. */
dlm_status dlm_commit(dlm_model* model, dlm_seq* const* seqs, int32_t n_seqs,
                      const float* conf, const int32_t* pred, const dlm_commit_rule* rule,
                      int32_t step, int32_t* n_committed, int32_t* n_masked, void* stream);

/* Forward over each request's finished canvas with the denoising mask; its K/V
 * are written to slots [T_r, T_r + C); then T_r += C.  No LM head.  A masked
 * position in a canvas sets DLM_DEVERR_MASK_APPEND on the device. */
dlm_status dlm_append_canvas(dlm_model* model, dlm_seq* const* seqs, int32_t n_seqs,
                             void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the same
 * denoising pass as dlm_denoise_step (same kernels, same results), with its
 * workspace taken from a static device array of DLM_STATIC_SCRATCH_BYTES that
 * the library holds on each device it runs on, from its first use there until
 * the process ends, instead of a caller-provided one.  The call allocates
 * nothing.  Every call on a device shares that device's array and leaves its
 * contents behind (no kernel of the pass reads scratch it has not written in
 * the same call, so nothing is cleared): calls that overlap on one device --
 * from two streams or two models -- race, and the caller must serialise them.
 * E_WORKSPACE (nothing enqueued) if the pass needs more than
 * DLM_STATIC_SCRATCH_BYTES, i.e. if dlm_workspace_bytes(model, n_seqs * C,
 * max T_r + C) exceeds it: the batch-1 canvases of the models this library
 * is built for need 50 to 100 MiB.  Other arguments and errors as
 * dlm_denoise_step. */
#define DLM_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
dlm_status dlm_denoise_step_noalloc(dlm_model* model, dlm_seq* const* seqs, int32_t n_seqs,
                                    float* conf, int32_t* pred, float* logits, void* stream);

/* Synchronises `stream`, reads and clears the device error word.  Returns
 * DLM_OK, or DLM_E_DEVICE with the bits in *bits (nullable). */
dlm_status dlm_check_device_status(dlm_model* model, void* stream, int32_t* bits);

/* Description of the last failure on the calling thread ("" if none). */
const char* dlm_last_error(void);

/* Test hook for MoE models.  While set, every forward also writes, for each
 * layer and each token row of the forward (device, nullable each):
 *   router_ids    int32 [n_layers][rows][top_k], the experts in selection order;
 *   router_logits fp32  [n_layers][rows][n_experts], the router logits.
 * capacity_rows: (layer, row) pairs the buffers hold; a forward needing more
 * (n_layers * rows) fails with E_CAPACITY before enqueuing anything. */
dlm_status dlm_debug_router(dlm_model* model, int32_t* router_ids, float* router_logits, int64_t capacity_rows);

/* Test hook: the per-token activation quantiser the fp8 models apply to every
 * GEMM A-operand.  x: device bf16 [rows, d]; q: device uint8 [rows, d] OCP
 * E4M3FN codes (out); s: device fp32 [rows] (out).  Per row: s = amax / 448
 * (1 for an all-zero row), q = nearest E4M3 value of x / s, ties to even,
 * saturating at +-448.  E_ARG on null pointers or rows / d < 1. */
dlm_status dlm_op_quant_rows(const void* x, int32_t rows, int32_t d, void* q, float* s, void* stream);

/* Test hook: one dense GEMM of the kind the model runs, C = A B^T, with A
 * [M, K] and B [N, K] row-major (device).  dtype DLM_F32, DLM_BF16 or DLM_FP8
 * (E4M3FN codes; then every product is scaled by a_scale[m] * b_scale[n], and
 * b2_scale[n] for B2 -- device fp32 arrays, required for DLM_FP8 only).
 *   swiglu = 0: C fp32 [M, N].
 *   swiglu = 1: C = silu(A B^T) * (A B2^T), bf16 (fp32 for DLM_F32) [M, N].
 * variant: tile shape, 0 = the one the model would pick, 1..12 forced (bf16
 * only), optionally or-ed with DLM_GEMM_B_TILED: B (and B2) are then in the
 * tiled weight layout of dlm_pack_weight; splits: split-K factor, 0 = the
 * model's choice.  ws / ws_bytes: room
 * for split-K partials (see dlm_op_gemm_workspace).  ms (host, nullable): when
 * set, the GEMM kernel is timed with events in its dispatch, the call
 * synchronises and writes the kernel's duration.  E_SHAPE unless K * element
 * size is a multiple of 128 bytes; E_ARG for a variant outside 0..12. */
#define DLM_GEMM_B_TILED 0x100
dlm_status dlm_op_gemm(int32_t dtype, int32_t swiglu, int32_t M, int32_t N, int32_t K, const void* A, const void* B,
                       const void* B2, const float* a_scale, const float* b_scale, const float* b2_scale, void* C,
                       void* ws, size_t ws_bytes, int32_t variant, int32_t splits, float* ms, void* stream);
size_t dlm_op_gemm_workspace(int32_t dtype, int32_t swiglu, int32_t M, int32_t N, int32_t K, int32_t variant,
                             int32_t splits);

/* Test hook: the MoE layer's grouped expert GEMM over MX weights (dtype
 * DLM_MXFP4 or DLM_MXFP6, else E_DTYPE).  E
 * experts, counts: HOST int32 [E], the rows of each (>= 0; M = their sum >= 1);
 * A: device bf16 [M, K], expert 0's rows first, then expert 1's, ...; B, S
 * (and B2, S2 for swiglu): the E experts' [N, K] matrices packed by
 * dlm_pack_mx.  swiglu = 0: C fp32 [M, N] = A B^T per expert; swiglu = 1:
 * C bf16 [M, N] = silu(A B^T) * (A B2^T).  B is decoded exactly (code value x
 * block scale); fp32 accumulation.  ws: device, dlm_op_mx_gemm_workspace(E)
 * bytes (the experts' row offsets and tile starts, copied from the host on
 * `stream`, which the call synchronises before the launch); variant: 0 = the model's tile shape, 1..5 forced; ms: as for
 * dlm_op_gemm.  E_ARG for null pointers, E outside [1, 256], a negative count,
 * M < 1 or a variant outside 0..5; E_SHAPE unless K % 128 == 0 and N >= 1;
 * E_WORKSPACE if ws_bytes is too small. */
dlm_status dlm_op_mx_gemm(int32_t dtype, int32_t swiglu, int32_t E, const int32_t* counts, int32_t N, int32_t K,
                          const void* A, const void* B, const void* S, const void* B2, const void* S2, void* C,
                          void* ws, size_t ws_bytes, int32_t variant, float* ms, void* stream);
size_t dlm_op_mx_gemm_workspace(int32_t E);

/* Test hook: the MoE layer's sort of (row, slot) assignments by expert.
 * ids: HOST int32 [n_assign], expert of each assignment (validated: each in
 * [0, E), else E_ARG; copied into ws on `stream`).  Outputs (device):
 * offs int32 [E + 1] (first sorted position of each expert, offs[E] =
 * n_assign), tile_start int32 [E + 1] (first bm-row tile of each expert, last
 * = total tiles), sorted_assign int32 [n_assign] (assignment indices ordered
 * by (expert, index)), inv int32 [n_assign] (sorted position of each
 * assignment).  Up to 4096 assignments one workgroup sorts them, beyond that
 * three kernels -- the two paths the model takes.  ws / ws_bytes: device
 * workspace of dlm_op_route_workspace(n_assign, E) bytes (E_WORKSPACE if
 * smaller).  E_ARG for null pointers, n_assign < 1, E outside [1, 256] or
 * bm < 1. */
dlm_status dlm_op_route(const int32_t* ids, int32_t n_assign, int32_t E, int32_t bm, int32_t* offs,
                        int32_t* tile_start, int32_t* sorted_assign, int32_t* inv, void* ws, size_t ws_bytes,
                        void* stream);
size_t dlm_op_route_workspace(int32_t n_assign, int32_t E);

/* Test hook: the MoE router's selection.  logits: device fp32 [rows, E];
 * ids: device int32 [rows, k] (out), the k experts with the largest logits in
 * decreasing order, ties to the lower expert id; w: device fp32 [rows, k]
 * (out), their softmax probabilities renormalised over the k.  E_ARG for null
 * pointers, rows < 1, E outside [1, 256] or k outside [1, min(16, E)]. */
dlm_status dlm_op_router_topk(const float* logits, int32_t rows, int32_t E, int32_t k, int32_t* ids, float* w,
                              void* stream);

/* Kernel timing.  `kernel_mask` bit i enables timing of kernel id i (0 = off):
 * every launch of a timed kernel is bracketed by HIP events on its stream.
 * dlm_timing_read synchronises, sums the elapsed times per kernel id since the
 * last read, and resets.
 *   ms[DLM_K_COUNT], launches[DLM_K_COUNT] (host, out; nullable).
 * DLM_K_COMBINE is kept for numbering only: the MoE layer's combine is part of
 * the RMSNorm that reads its result (DLM_K_NORM). */
typedef enum {
    DLM_K_EMBED = 0, DLM_K_NORM, DLM_K_GEMM_QKV, DLM_K_ROPE_KV, DLM_K_ATTN,
    DLM_K_ATTN_MERGE, DLM_K_GEMM_O, DLM_K_GEMM_GATE_UP, DLM_K_GEMM_DOWN,
    DLM_K_QUANT, DLM_K_ROUTER, DLM_K_TOPK, DLM_K_PERMUTE, DLM_K_EXPERT_GATE_UP,
    DLM_K_EXPERT_DOWN, DLM_K_COMBINE, DLM_K_LM_HEAD, DLM_K_LM_MERGE, DLM_K_COMMIT,
    DLM_K_SPLITK_EPILOGUE,
    DLM_K_COUNT
} dlm_kernel_id;
dlm_status dlm_timing_enable(dlm_model* model, int32_t kernel_mask);
dlm_status dlm_timing_read(dlm_model* model, float* ms, int32_t* launches);
const char* dlm_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* DLM_H */
