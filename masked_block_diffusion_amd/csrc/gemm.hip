// MFMA GEMMs for gfx950: C = A * B^T with A [M, K] and B [N, K] both K-contiguous
// (a token-major activation times a row-major [out, in] weight), fp32
// accumulation, and the epilogues the transformer needs fused in:
//   store fp32 / bf16, residual add into the fp32 stream, SwiGLU over two weight
//   matrices (gate and up) sharing one A tile, and the LM-head reduction that
//   turns each (row, vocab tile) into (max, lowest argmax, sum exp(l - max)).
// A grouped variant runs one GEMM per expert over the token rows routed to it,
// gathering A rows through the permutation.
//
// Tiling: a 256-thread workgroup (4 waves) owns a BM x BN output tile; A and B
// K-tiles of 128 bytes per row are staged through LDS (double-buffered, the next
// tile prefetched into registers while the current one feeds the MFMAs).  Each
// wave owns a (BM/WM) x (BN/WN) sub-tile of 16x16 MFMA blocks.  The workgroup
// order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs, so the
// linear tile index is remapped to give each XCD a contiguous range of
// (n-tile, m-tile) pairs, n-major, so that the m-tiles reading one weight tile
// run together on one XCD and share its L2.
#include "common.h"
#include "kernels.h"

namespace dlm {

enum Epi { EPI_F32 = 0, EPI_BF16, EPI_ADD_F32, EPI_SWIGLU_BF16, EPI_SWIGLU_F32, EPI_LMHEAD };

constexpr int BKB = 128;             // K bytes per pipeline stage
constexpr int LDS_ROW = BKB + 16;    // padded LDS row (bytes)

template <int BM, int BN, bool DUAL>
struct Smem {
    static constexpr int A = BM * LDS_ROW;
    static constexpr int B = BN * LDS_ROW;
    static constexpr int STAGE = A + B * (DUAL ? 2 : 1);
    static constexpr int BYTES = 2 * STAGE;
};

// Per-thread 16-byte chunks of a tile with R rows: chunk c = tid + 256 j covers
// row c / 8, bytes (c % 8) * 16.
template <int R> struct Chunks { static constexpr int N = (R * 8 + 255) / 256; };

struct TileRows {
    // Address of each chunk row (or null when the row is outside the matrix).
    const uint8_t* p;
};

template <typename T, int BM, int BN, int WM, int WN, bool DUAL>
struct Core {
    static constexpr int TM = BM / WM / 16;
    static constexpr int TN = BN / WN / 16;
    static constexpr int KSB = Mfma<T>::KSTEP * (int)sizeof(T);   // bytes per MFMA k-step
    static constexpr int LB = Mfma<T>::LANE_BYTES;
    static constexpr int AC = Chunks<BM>::N;
    static constexpr int BC = Chunks<BN>::N;
    typedef typename Mfma<T>::frag frag;
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile");
    static_assert(WM * WN == 4, "4 waves");

    const uint8_t* arow[AC];
    const uint8_t* brow[BC];
    const uint8_t* b2row[BC];
    u32x4 ra[AC], rb[BC], rb2[BC];
    f32x4 acc[TM][TN];
    f32x4 acc2[DUAL ? TM : 1][DUAL ? TN : 1];
    long kbytes;

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (DUAL) acc2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
    }

    __device__ __forceinline__ void load(int kt) {
        const int tid = threadIdx.x;
        const long kb = (long)kt * BKB + (tid % 8) * 16;
        const bool kin = kb < kbytes;
#pragma unroll
        for (int j = 0; j < AC; ++j) {
            const uint8_t* p = arow[j];
            ra[j] = (p && kin) ? *(const u32x4*)(p + kb) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < BC; ++j) {
            const uint8_t* p = brow[j];
            rb[j] = (p && kin) ? __builtin_nontemporal_load((const u32x4*)(p + kb)) : u32x4{0, 0, 0, 0};
            if constexpr (DUAL) {
                const uint8_t* p2 = b2row[j];
                rb2[j] = (p2 && kin) ? __builtin_nontemporal_load((const u32x4*)(p2 + kb)) : u32x4{0, 0, 0, 0};
            }
        }
    }

    __device__ __forceinline__ void store(uint8_t* stage) {
        const int tid = threadIdx.x;
        uint8_t* sa = stage;
        uint8_t* sb = stage + Smem<BM, BN, DUAL>::A;
        uint8_t* sb2 = sb + Smem<BM, BN, DUAL>::B;
#pragma unroll
        for (int j = 0; j < AC; ++j) {
            const int c = tid + 256 * j;
            if (c < BM * 8) *(u32x4*)(sa + (c / 8) * LDS_ROW + (c % 8) * 16) = ra[j];
        }
#pragma unroll
        for (int j = 0; j < BC; ++j) {
            const int c = tid + 256 * j;
            if (c < BN * 8) {
                *(u32x4*)(sb + (c / 8) * LDS_ROW + (c % 8) * 16) = rb[j];
                if constexpr (DUAL) *(u32x4*)(sb2 + (c / 8) * LDS_ROW + (c % 8) * 16) = rb2[j];
            }
        }
    }

    __device__ __forceinline__ void compute(const uint8_t* stage) {
        const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
        const int wm = wave / WN, wn = wave % WN;
        const uint8_t* sa = stage + (wm * (BM / WM) + lane % 16) * LDS_ROW + (lane / 16) * LB;
        const uint8_t* sb = stage + Smem<BM, BN, DUAL>::A + (wn * (BN / WN) + lane % 16) * LDS_ROW + (lane / 16) * LB;
#pragma unroll
        for (int s = 0; s < BKB / KSB; ++s) {
            frag af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = *(const frag*)(sa + i * 16 * LDS_ROW + s * KSB);
#pragma unroll
            for (int j = 0; j < TN; ++j) bf[j] = *(const frag*)(sb + j * 16 * LDS_ROW + s * KSB);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = Mfma<T>::mma(af[i], bf[j], acc[i][j]);
            if constexpr (DUAL) {
                frag bf2[TN];
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bf2[j] = *(const frag*)(sb + Smem<BM, BN, DUAL>::B + j * 16 * LDS_ROW + s * KSB);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) acc2[i][j] = Mfma<T>::mma(af[i], bf2[j], acc2[i][j]);
            }
        }
    }

    __device__ __forceinline__ void run(uint8_t* smem) {
        zero();
        const int nkt = (int)((kbytes + BKB - 1) / BKB);
        load(0);
        store(smem);
        __syncthreads();
        for (int kt = 0; kt < nkt; ++kt) {
            uint8_t* cur = smem + (kt & 1) * Smem<BM, BN, DUAL>::STAGE;
            uint8_t* nxt = smem + ((kt + 1) & 1) * Smem<BM, BN, DUAL>::STAGE;
            if (kt + 1 < nkt) load(kt + 1);
            compute(cur);
            if (kt + 1 < nkt) store(nxt);
            __syncthreads();
        }
    }
};

// Remap a linear workgroup id so each XCD (id % 8) gets a contiguous range.
__device__ __forceinline__ int xcd_remap(int b, int total) {
    if (total % 8 != 0) return b;
    return (b % 8) * (total / 8) + b / 8;
}

struct EpiArgs {
    int epi;
    void* C; long ldc;                   // elements
    const float* a_scale;                // fp8: per A-source-row
    const float* b_scale;                // fp8: per output column
    const float* b2_scale;
    // LM head
    float* pmax; float* psum; int* pidx; int n_tiles; int mask_col;
    float* logits; long ld_logits;
};

// Applies the epilogue to one wave's accumulators.  rows/cols are global
// indices; srow[i] = A source row (for per-token scales), M/N bounds.
template <typename T, int BM, int BN, int WM, int WN, bool DUAL, int EPI>
__device__ __forceinline__ void epilogue(Core<T, BM, BN, WM, WN, DUAL>& c, const EpiArgs& e,
                                         int m0, int n0, int mlim, int N, const int* gather,
                                         int gather_div, int ntile) {
    typedef Core<T, BM, BN, WM, WN, DUAL> C;
    const int lane = threadIdx.x % WAVE, wave = threadIdx.x / WAVE;
    const int wm = wave / WN, wn = wave % WN;
    const int rbase = m0 + wm * (BM / WM) + 4 * (lane / 16);
    const int cbase = n0 + wn * (BN / WN) + lane % 16;
    if constexpr (EPI == EPI_LMHEAD) {
        static_assert(WN == 1, "LM head epilogue needs whole-tile columns per wave");
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = rbase + i * 16 + v;
                const bool rok = row < mlim;
                float sa = 1.f;
                if constexpr (sizeof(T) == 1) sa = rok ? e.a_scale[row] : 1.f;
                float vals[C::TN];
                float mx = -INFINITY;
                int ix = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const int col = cbase + j * 16;
                    float x = c.acc[i][j][v];
                    if constexpr (sizeof(T) == 1) x *= sa * (col < N ? e.b_scale[col] : 0.f);
                    if (rok && e.logits && col < N) e.logits[(long)row * e.ld_logits + col] = x;
                    if (col >= N || col == e.mask_col) x = -INFINITY;
                    vals[j] = x;
                    if (x > mx) { mx = x; ix = col; }
                }
                // across the 16 lanes holding this row's columns; ties -> lower column
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) {
                    const float om = __shfl_xor(mx, o, WAVE);
                    const int oi = __shfl_xor(ix, o, WAVE);
                    if (om > mx || (om == mx && oi < ix)) { mx = om; ix = oi; }
                }
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < C::TN; ++j) s += (vals[j] == -INFINITY) ? 0.f : __expf(vals[j] - mx);
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, WAVE);
                if (rok && lane % 16 == 0) {
                    const long k = (long)row * e.n_tiles + ntile;
                    e.pmax[k] = mx;
                    e.psum[k] = s;
                    e.pidx[k] = ix;
                }
            }
        return;
    } else {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = rbase + i * 16 + v;
                if (row >= mlim) continue;
                float sa = 1.f;
                if constexpr (sizeof(T) == 1) {
                    const int src = gather ? gather[row] / gather_div : row;
                    sa = e.a_scale[src];
                }
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const int col = cbase + j * 16;
                    if (col >= N) continue;
                    float x = c.acc[i][j][v];
                    if constexpr (sizeof(T) == 1) x *= sa * e.b_scale[col];
                    const long off = (long)row * e.ldc + col;
                    if constexpr (EPI == EPI_F32) {
                        ((float*)e.C)[off] = x;
                    } else if constexpr (EPI == EPI_BF16) {
                        ((bf16_t*)e.C)[off] = f32_to_bf16(x);
                    } else if constexpr (EPI == EPI_ADD_F32) {
                        ((float*)e.C)[off] += x;
                    } else if constexpr (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_F32) {
                        float u = c.acc2[i][j][v];
                        if constexpr (sizeof(T) == 1) u *= sa * e.b2_scale[col];
                        const float y = silu_f(x) * u;
                        if constexpr (EPI == EPI_SWIGLU_BF16) ((bf16_t*)e.C)[off] = f32_to_bf16(y);
                        else ((float*)e.C)[off] = y;
                    }
                }
            }
    }
}

struct DenseArgs {
    const uint8_t* A; long lda;          // bytes
    const uint8_t* B; const uint8_t* B2; long ldb;
    int M, N, K;
    EpiArgs e;
};

template <typename T, int BM, int BN, int WM, int WN, bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_dense_kernel(DenseArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<BM, BN, DUAL>::BYTES];
    const int mt_n = (a.M + BM - 1) / BM, nt_n = (a.N + BN - 1) / BN;
    const int lin = xcd_remap(blockIdx.x, mt_n * nt_n);
    const int nt = lin / mt_n, mt = lin % mt_n;
    const int m0 = mt * BM, n0 = nt * BN;
    Core<T, BM, BN, WM, WN, DUAL> c;
    c.kbytes = (long)a.K * sizeof(T);
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < Core<T, BM, BN, WM, WN, DUAL>::AC; ++j) {
        const int r = (tid + 256 * j) / 8 + m0;
        c.arow[j] = (r < a.M && tid + 256 * j < BM * 8) ? a.A + (long)r * a.lda : nullptr;
    }
#pragma unroll
    for (int j = 0; j < Core<T, BM, BN, WM, WN, DUAL>::BC; ++j) {
        const int r = (tid + 256 * j) / 8 + n0;
        const bool ok = r < a.N && tid + 256 * j < BN * 8;
        c.brow[j] = ok ? a.B + (long)r * a.ldb : nullptr;
        if constexpr (DUAL) c.b2row[j] = ok ? a.B2 + (long)r * a.ldb : nullptr;
    }
    c.run(smem);
    epilogue<T, BM, BN, WM, WN, DUAL, EPI>(c, a.e, m0, n0, a.M, a.N, nullptr, 1, nt);
}

struct GroupedArgs {
    const uint8_t* A; long lda;          // bytes
    const int* gather; int gather_div;   // A row of permuted row p = gather[p] / gather_div (nullable)
    const uint8_t* B; const uint8_t* B2; long ldb; long b_stride;   // bytes between experts
    const float* b_scale; const float* b2_scale; long bs_stride;     // elements between experts
    const int* offs;        // [E + 1] permuted row offsets per expert
    const int* tile_start;  // [E + 1] first m-tile of each expert (for this BM)
    int E, max_mtiles, N, K;
    EpiArgs e;
};

template <typename T, int BM, int BN, int WM, int WN, bool DUAL, int EPI>
__global__ __launch_bounds__(256) void gemm_grouped_kernel(GroupedArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[Smem<BM, BN, DUAL>::BYTES];
    const int nt_n = (a.N + BN - 1) / BN;
    const int lin = xcd_remap(blockIdx.x, a.max_mtiles * nt_n);
    const int nt = lin / a.max_mtiles, mt = lin % a.max_mtiles;
    if (mt >= a.tile_start[a.E]) return;
    // expert owning m-tile mt: last e with tile_start[e] <= mt
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int ex = lo;
    const int m0 = a.offs[ex] + (mt - a.tile_start[ex]) * BM;
    const int mlim = a.offs[ex + 1];
    const int n0 = nt * BN;
    Core<T, BM, BN, WM, WN, DUAL> c;
    c.kbytes = (long)a.K * sizeof(T);
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < Core<T, BM, BN, WM, WN, DUAL>::AC; ++j) {
        const int r = (tid + 256 * j) / 8 + m0;
        const bool ok = r < mlim && tid + 256 * j < BM * 8;
        const int src = ok ? (a.gather ? a.gather[r] / a.gather_div : r) : 0;
        c.arow[j] = ok ? a.A + (long)src * a.lda : nullptr;
    }
    const uint8_t* Be = a.B + (long)ex * a.b_stride;
    const uint8_t* B2e = DUAL ? a.B2 + (long)ex * a.b_stride : nullptr;
#pragma unroll
    for (int j = 0; j < Core<T, BM, BN, WM, WN, DUAL>::BC; ++j) {
        const int r = (tid + 256 * j) / 8 + n0;
        const bool ok = r < a.N && tid + 256 * j < BN * 8;
        c.brow[j] = ok ? Be + (long)r * a.ldb : nullptr;
        if constexpr (DUAL) c.b2row[j] = ok ? B2e + (long)r * a.ldb : nullptr;
    }
    c.run(smem);
    EpiArgs e = a.e;
    if constexpr (sizeof(T) == 1) {
        e.b_scale = a.b_scale + (long)ex * a.bs_stride;
        if constexpr (DUAL) e.b2_scale = a.b2_scale + (long)ex * a.bs_stride;
    }
    epilogue<T, BM, BN, WM, WN, DUAL, EPI>(c, e, m0, n0, mlim, a.N, a.gather, a.gather_div, nt);
}

// ------------------------------------------------------------- launchers --

template <typename T, int BM, int BN, int WM, int WN, bool DUAL, int EPI>
static void launch_dense(const GemmDesc& d, hipStream_t st) {
    DenseArgs a;
    a.A = (const uint8_t*)d.A; a.lda = d.lda * (long)sizeof(T);
    a.B = (const uint8_t*)d.B; a.B2 = (const uint8_t*)d.B2; a.ldb = d.ldb * (long)sizeof(T);
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.e.epi = EPI; a.e.C = d.C; a.e.ldc = d.ldc;
    a.e.a_scale = d.a_scale; a.e.b_scale = d.b_scale; a.e.b2_scale = d.b2_scale;
    a.e.pmax = d.pmax; a.e.psum = d.psum; a.e.pidx = d.pidx; a.e.n_tiles = (d.N + BN - 1) / BN;
    a.e.mask_col = d.mask_col; a.e.logits = d.logits; a.e.ld_logits = d.ld_logits;
    const int grid = ((d.M + BM - 1) / BM) * ((d.N + BN - 1) / BN);
    if (grid == 0) return;
    hipLaunchKernelGGL((gemm_dense_kernel<T, BM, BN, WM, WN, DUAL, EPI>), dim3(grid), dim3(256), 0, st, a);
}

template <typename T, int BM, int BN, int WM, int WN, bool DUAL, int EPI>
static void launch_grouped(const GemmDesc& d, hipStream_t st) {
    GroupedArgs a;
    a.A = (const uint8_t*)d.A; a.lda = d.lda * (long)sizeof(T);
    a.gather = d.gather; a.gather_div = d.gather_div;
    a.B = (const uint8_t*)d.B; a.B2 = (const uint8_t*)d.B2; a.ldb = d.ldb * (long)sizeof(T);
    a.b_stride = d.b_stride * (long)sizeof(T);
    a.b_scale = d.b_scale; a.b2_scale = d.b2_scale; a.bs_stride = d.bs_stride;
    a.offs = d.offs; a.tile_start = d.tile_start; a.E = d.E; a.N = d.N; a.K = d.K;
    a.max_mtiles = (d.M + BM - 1) / BM + d.E;
    a.e.epi = EPI; a.e.C = d.C; a.e.ldc = d.ldc;
    a.e.a_scale = d.a_scale; a.e.b_scale = nullptr; a.e.b2_scale = nullptr;
    a.e.pmax = nullptr; a.e.psum = nullptr; a.e.pidx = nullptr; a.e.n_tiles = 0;
    a.e.mask_col = -1; a.e.logits = nullptr; a.e.ld_logits = 0;
    const int grid = a.max_mtiles * ((d.N + BN - 1) / BN);
    if (d.M == 0 || grid == 0) return;
    hipLaunchKernelGGL((gemm_grouped_kernel<T, BM, BN, WM, WN, DUAL, EPI>), dim3(grid), dim3(256), 0, st, a);
}

// Tile shapes.  Small-M problems (the tiny model's canvas) use 32-row tiles;
// canvas-sized M (256 rows per request) 128 x 64; prefill-sized M 128 x 128.
template <typename T, bool DUAL, int EPI>
static void dispatch_dense(const GemmDesc& d, hipStream_t st) {
    if constexpr (EPI == EPI_LMHEAD) {
        if (d.M <= 64) launch_dense<T, 64, 64, 4, 1, false, EPI>(d, st);
        else launch_dense<T, 128, 64, 4, 1, false, EPI>(d, st);
    } else if constexpr (DUAL) {
        if (d.M <= 64) launch_dense<T, 32, 64, 1, 4, true, EPI>(d, st);
        else launch_dense<T, 128, 64, 2, 2, true, EPI>(d, st);
    } else {
        if (d.M <= 64) launch_dense<T, 32, 64, 1, 4, false, EPI>(d, st);
        else if (d.M <= 512) launch_dense<T, 128, 64, 2, 2, false, EPI>(d, st);
        else launch_dense<T, 128, 128, 2, 2, false, EPI>(d, st);
    }
}

template <typename T>
static void gemm_t(const GemmDesc& d, hipStream_t st) {
    switch (d.epi) {
        case GEMM_STORE_F32: dispatch_dense<T, false, EPI_F32>(d, st); break;
        case GEMM_STORE_BF16: dispatch_dense<T, false, EPI_BF16>(d, st); break;
        case GEMM_ADD_F32: dispatch_dense<T, false, EPI_ADD_F32>(d, st); break;
        case GEMM_SWIGLU:
            if (d.out_f32) dispatch_dense<T, true, EPI_SWIGLU_F32>(d, st);
            else dispatch_dense<T, true, EPI_SWIGLU_BF16>(d, st);
            break;
        case GEMM_LMHEAD: dispatch_dense<T, false, EPI_LMHEAD>(d, st); break;
    }
}

template <typename T>
static void grouped_t(const GemmDesc& d, hipStream_t st) {
    // one tile row count for both expert GEMMs: GROUPED_BM (the routing scan
    // computes each expert's first m-tile for this BM)
    switch (d.epi) {
        case GEMM_SWIGLU:
            if (d.out_f32) launch_grouped<T, GROUPED_BM, 64, 1, 4, true, EPI_SWIGLU_F32>(d, st);
            else launch_grouped<T, GROUPED_BM, 64, 1, 4, true, EPI_SWIGLU_BF16>(d, st);
            break;
        case GEMM_STORE_F32: launch_grouped<T, GROUPED_BM, 64, 1, 4, false, EPI_F32>(d, st); break;
        default: break;
    }
}

void gemm(const GemmDesc& d, hipStream_t st) {
    switch (d.dtype) {
        case DT_F32: gemm_t<float>(d, st); break;
        case DT_BF16: gemm_t<bf16_t>(d, st); break;
        case DT_FP8: gemm_t<fp8_t>(d, st); break;
    }
}

void gemm_grouped(const GemmDesc& d, hipStream_t st) {
    switch (d.dtype) {
        case DT_F32: grouped_t<float>(d, st); break;
        case DT_BF16: grouped_t<bf16_t>(d, st); break;
        case DT_FP8: grouped_t<fp8_t>(d, st); break;
    }
}

int lm_head_tile_n() { return 64; }

}  // namespace dlm
