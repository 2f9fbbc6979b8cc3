// Host-side launchers of the gfx950 kernels.  Every launcher enqueues on the
// given stream and returns immediately; shapes are validated by the caller.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlm {

// Kernel timing: while a LaunchTimer is armed on this thread, the next kernel
// launched through launch() carries its start / stop events in its own
// dispatch (hipExtLaunchKernelGGL), so the elapsed time is that kernel's
// execution, without separate marker packets around it.
struct LaunchTimer {
    hipEvent_t start = nullptr, stop = nullptr;
    bool armed = false;
};
LaunchTimer*& launch_timer();

template <typename... KArgs, typename... Args>
inline void launch(void (*k)(KArgs...), dim3 grid, dim3 block, uint32_t shm, hipStream_t st, Args... args) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    LaunchTimer* t = launch_timer();
    if (t && t->armed) {
        t->armed = false;
        e0 = t->start;
        e1 = t->stop;
    }
    hipExtLaunchKernelGGL(k, grid, block, shm, st, e0, e1, 0, args...);
}

enum DType { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

enum GemmEpi { GEMM_STORE_F32 = 0, GEMM_STORE_BF16, GEMM_ADD_F32, GEMM_SWIGLU, GEMM_LMHEAD };

constexpr int MAX_SEQS = 64;

// m-tile rows of the grouped (per-expert) GEMMs for operand type `dtype` and
// n_assign (row, expert) assignments over E experts (the GEMM's M and E); the
// routing scan computes each expert's first m-tile for this tile height.
int grouped_bm(int dtype, int n_assign, int E);
// True when the experts average 256 rows or more (the compute-bound tile
// family): many requests' canvases, prompts.
bool grouped_compute_bound(int n_assign, int E);

// C[M, N] (op)= A[M, K] * B[N, K]^T.  Leading dimensions in elements.
struct GemmDesc {
    int dtype = DT_BF16;        // element type of A and B
    int epi = GEMM_STORE_F32;
    bool out_f32 = false;       // SwiGLU output in fp32 (f32 models) instead of bf16
    const void* A = nullptr; long lda = 0;
    const void* B = nullptr; const void* B2 = nullptr; long ldb = 0;
    // B / B2 in the tiled weight layout (blocks of 16 rows x 128 bytes of K,
    // see dlm_pack_weight); ldb is then unused
    bool b_tiled = false;
    const float* a_scale = nullptr;   // fp8: per A row
    const float* b_scale = nullptr;   // fp8: per output column (B row)
    const float* b2_scale = nullptr;
    int M = 0, N = 0, K = 0;
    void* C = nullptr; long ldc = 0;
    // LM head reduction: partials [M, ceil(N / lm_head_tile_n(M))]
    float* pmax = nullptr; float* psum = nullptr; int* pidx = nullptr;
    int mask_col = -1;
    float* logits = nullptr; long ld_logits = 0;
    // grouped
    const int* gather = nullptr; int gather_div = 1;
    long b_stride = 0;          // elements between experts' B matrices
    long bs_stride = 0;         // elements between experts' scale vectors
    const int* offs = nullptr;  // [E + 1]
    const int* tile_start = nullptr;  // [E + 1]
    int E = 0;
    // split-K (dense GEMMs): fp32 partials [splits][M][N] (x2 for SwiGLU)
    float* splitk = nullptr; long splitk_floats = 0;
    // forced tile variant (1..gemm_variants(); bf16 store / SwiGLU only) and split factor; 0 = chosen by shape
    int variant = 0;
    int force_splits = 0;
};
int gemm_variants();

// Tiled weight layout (what the model's projection GEMMs read): a [N, K]
// matrix of eb-byte elements as blocks of 16 rows x 128 bytes of K; block
// (g, kt) at byte (g * nkt + kt) * 2048 with nkt = K * eb / 128, row n % 16
// of block g = n / 16 at +128 * (n % 16) inside it.  N is padded to a
// multiple of 16 (zero rows); a batch of matrices (experts) is consecutive.
long packed_rows(int N);
long packed_weight_bytes(int eb, int batch, int N, int K);
void pack_weight(int eb, int batch, int N, int K, const void* src, void* dst, hipStream_t st);

// Dense and grouped GEMMs.  K * element size must be a multiple of 128 bytes.
// gemm_main launches the GEMM and returns its split-K factor; when that is
// above 1, gemm_splitk_finish(d, splits) must follow on the same stream (it
// sums the partials in split order and applies the epilogue).
int gemm_main(const GemmDesc& d, hipStream_t st);
void gemm_splitk_finish(const GemmDesc& d, int splits, hipStream_t st);
void gemm_grouped(const GemmDesc& d, hipStream_t st);
// fp32 partial space the dense GEMM d uses for split-K (0 if unsplit)
long gemm_splitk_floats(const GemmDesc& d);
// vocab columns per LM-head tile (one partial per row and tile) for M rows;
// the narrowest tile is used for M <= 64
int lm_head_tile_n(int M);

// MX expert weights (mx.hip): MXFP4 (E2M1, bits = 4) and MXFP6 (E2M3, bits =
// 6).  Packed layout of a [N, K] matrix (K a multiple of 128, N padded to a
// multiple of 16): codes in blocks of 16 rows x RB bytes (RB = 128 * bits / 8,
// the row-major code bytes of 128 elements), block (g, t) at byte (g * K / 128
// + t) * 16 RB; E8M0 scales in blocks of 64 bytes, block (g, t) at byte (g * K
// / 128 + t) * 64, byte r + 16 j = row 16 g + r, elements 128 t + 32 j .. + 32.
// Matrices of a batch follow one another.
long mx_code_bytes(int bits, int N, int K);
long mx_scale_bytes(int N, int K);
// codes [batch, N, K * bits / 8] and scales [batch, N, K / 32] row-major -> packed
void mx_pack(int bits, int batch, int N, int K, const void* codes, const void* scales, void* dst_codes,
             void* dst_scales, hipStream_t st);
// m-tile rows of the MX grouped GEMM (the routing's tile height for it)
int mx_grouped_bm();
// Grouped expert GEMM with bf16 A [M, K] (rows in expert order, or gathered as
// in GemmDesc) and MX B: swiglu -> C bf16 = silu(A B^T) * (A B2^T), else
// C fp32 = A B^T.  offs / tile_start as for gemm_grouped with mx_grouped_bm().
struct MxDesc {
    int bits = 4;                                 // 4: MXFP4 (E2M1), 6: MXFP6 (E2M3)
    bool swiglu = false;
    const void* A = nullptr; long lda = 0;        // elements
    const int* gather = nullptr; int gather_div = 1;
    const void* B = nullptr; const void* B2 = nullptr;
    const void* S = nullptr; const void* S2 = nullptr;
    long b_stride = 0, s_stride = 0;              // bytes between experts
    const int* offs = nullptr; const int* tile_start = nullptr;
    int E = 0, M = 0, N = 0, K = 0;
    void* C = nullptr; long ldc = 0;              // elements
    int variant = 0;                              // 0 = default tile shape, 1..mx_variants() forced
};
void mx_grouped(const MxDesc& d, hipStream_t st);
int mx_variants();

// Token ids of one forward: one flat array, or per-request canvases.
struct IdSource {
    const int32_t* flat;               // nullable
    const int32_t* canvas[MAX_SEQS];   // per request (when flat is null)
    int per_seq;                       // rows per request
};

// Requests of one forward: KV cache base, cached tokens T and capacity.
// Tokens per KV page (the attention kernel's key tile).
constexpr int KV_PAGE = 64;

// The requests of one forward and their caches (layout in kvcache.h).
struct SeqTab {
    void* kv[MAX_SEQS];          // contiguous cache, or the page pool's base
    const int* pt[MAX_SEQS];     // page table (device), NULL for a contiguous cache
    int T[MAX_SEQS];
    int cap[MAX_SEQS];           // capacity (tokens) of each request's cache
    long page_elems;             // elements per page: n_layers * 2 * n_kv_heads * KV_PAGE * head_dim
    int n;
    int per_seq;                 // rows per request in this forward
};

// x[r] = float(embed[id_r]); ids outside [0, vocab) set DEVERR_TOKEN_RANGE
// (and read row 0); with check_mask, ids equal to mask_id set DEVERR_MASK_APPEND.
void embed(const IdSource& ids, int rows, const void* table, int dtype, int d, int vocab,
           int mask_id, bool check_mask, float* x, int* err, hipStream_t st);

// A GEMM result [rows, cols] as its consumer reads it: the direct fp32 output
// (splits = 1, no scales) or split-K partials p[s * stride + row * cols + col],
// s < splits, times a_scale[row] * b_scale[col] when the scales are set (fp8).
struct Partials {
    const float* p = nullptr;
    int splits = 1;
    long stride = 0;
    const float* a_scale = nullptr;
    const float* b_scale = nullptr;
};

// The routed experts' part of an MoE layer's output, for row r:
// sum over slots s (in selection order) of w[r * k + s] * y[inv[r * k + s]]
// (y [assignments, d] in sorted order: bf16 when y_bf16, else fp32).  Unset
// when y is null.
struct MoeGather {
    const void* y = nullptr;
    const int* inv = nullptr;
    const float* w = nullptr;
    int k = 0;
    bool y_bf16 = false;
};

// x += res + moe (the residual update of a split O / down projection when
// res.p is set, then the MoE layer's routed experts when moe.y is set -- the
// shared expert arriving as res), then h = x / sqrt(mean(x^2) + eps) * g per
// row, written to every non-null output: hf fp32, hb bf16, and (fp8 models) hq
// E4M3 codes with per-row scales hs quantised from the bf16 value.
// d <= rmsnorm_max_dim(), d % 4 == 0.
int rmsnorm_max_dim();
void rmsnorm(float* x, const Partials& res, const MoeGather& moe, const float* g, int rows, int d, float eps,
             float* hf, uint16_t* hb, uint8_t* hq, float* hs, hipStream_t st);

// Per-row E4M3 quantisation of a bf16 matrix [rows, d]: s = amax / 448 (1 for a
// zero row), q = e4m3(x / s).
void quant_rows(const uint16_t* x, int rows, int d, uint8_t* q, float* s, hipStream_t st);

// RoPE on Q and K of qkv ([rows, (Hq + 2 Hkv) * dh], see Partials) at absolute
// positions T_r + i; Q -> q_out [rows, Hq * dh]; K, V -> cache slots T_r + i of
// layer l.  Element type of q_out and the cache: fp32 (f32 models) or bf16.
void rope_kv(const Partials& qkv, int rows, const SeqTab& seqs, int layer, int n_layers, int hq,
             int hkv, int dh, float base, bool f32, void* q_out, hipStream_t st);

// Attention of rows' queries (q [rows, Hq * dh]) over request r's cache slots
// [0, T_r + per_seq): causal (prefill: key t visible to the query at position
// p iff t <= p) or block (every key visible).  out [rows, Hq * dh].
struct AttnWork {
    float* o_part;      // split-KV partial outputs
    float* ml_part;     // split-KV partial (max, sum)
    long capacity;      // floats available in o_part
    LaunchTimer* merge_timer;   // timer for the split-KV merge kernel (nullable)
};
void attention(const void* q, const SeqTab& seqs, int layer, int n_layers, int hq, int hkv,
               int dh, bool causal, bool f32, void* out, const AttnWork& w, hipStream_t st);
long attention_work_floats(int rows, int hq, int dh);

// Router: logits fp32 [rows, E] (the router GEMM's output or its split-K
// partials, no scales) -> top-k experts (ties -> lower id), weights = softmax
// probabilities renormalised over the chosen k.
void router_topk(const Partials& logits, int rows, int E, int k, int* ids, float* w, int* ids_copy,
                 float* logits_copy, hipStream_t st);

// Stable counting sort of the rows*k assignments by expert: offs [E + 1],
// tile_start [E + 1] (bm-row tiles, bm = grouped_bm), sorted_assign [A] (assignment
// index a = row * k + slot, ordered by (expert, a)), inv [A] (position of a).
struct RouteWork { int* hist; int* local_rank; };   // hist [blocks * E], local_rank [A]
void moe_route(const int* ids, int n_assign, int E, int bm, int* offs, int* tile_start, int* sorted_assign,
               int* inv, const RouteWork& w, hipStream_t st);
int route_blocks(int n_assign);


// LM-head partials (max, sum exp, argmax) per (row, vocab tile) -> conf = 1/Z,
// pred = lowest argmax.
void lm_merge(const float* pmax, const float* psum, const int* pidx, int rows, int n_tiles,
              float* conf, int* pred, hipStream_t st);

// Commit (one workgroup per request).  kind 0: top-k with k; kind 1: threshold
// (all masked with conf >= thr, at least the most confident one); force_all:
// every masked position.  edit_thr > 0: token editing -- every position that
// held a token, whose prediction differs and whose conf >= edit_thr, takes its
// prediction.  n_committed counts commits plus edits.
void commit(int32_t* const* canvases, int n_seqs, int C, const float* conf, const int* pred,
            int mask_id, int kind, int k, float thr, bool force_all, float edit_thr, int* n_committed,
            int* n_masked, hipStream_t st);

}  // namespace dlm
