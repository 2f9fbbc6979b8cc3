// MFMA GEMMs for gfx950: C = A * B^T with A [M, K] and B [N, K] both K-contiguous
// (a token-major activation times a row-major [out, in] weight), fp32
// accumulation, and the epilogues the transformer needs fused in:
//   store fp32 / bf16, residual add into the fp32 stream, SwiGLU over two weight
//   matrices (gate and up) sharing one A tile, and the LM-head reduction that
//   turns each (row, vocab tile) into (max, lowest argmax, sum exp(l - max)).
// A grouped variant runs one GEMM per expert over the token rows routed to it,
// gathering A rows through the permutation.
//
// Data movement.  A 256-thread workgroup (4 waves) owns a BM x BN output tile.
// K advances in stages of 128 bytes per row; each stage (the A rows, then the B
// rows, then for SwiGLU the second weight's rows) is copied global -> LDS by
// global_load_lds_dwordx4, which writes each wave's 64 x 16 bytes straight into
// LDS without passing through registers.  NS stages are in flight at once (an
// LDS ring), so the weight stream keeps several tens of KB outstanding per CU
// -- what HBM latency needs at 8 TB/s.  One barrier per stage: wait for the
// stage's loads, barrier, refill the slot the previous stage used, then run the
// stage's MFMAs.  The 16-byte chunks of a row are XOR-swizzled by (row & 7) so
// the fragment reads of 16 consecutive rows spread over the LDS banks.
//
// Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs, so
// the linear tile index is remapped to give each XCD a contiguous range, in an
// order where the m-tiles reading one weight K-slice are adjacent (one L2).
//
// Weight-streaming shapes (a 256-row canvas against a 2048-wide projection)
// have too few output tiles for 256 CUs, so K is split across workgroups.
// Partial tiles go to the workspace with plain stores and a second kernel sums
// them in split order and applies the epilogue: deterministic, and no
// device-scope fences (which on this chip write back and invalidate L2).
#include "common.h"
#include "kernels.h"

namespace dlm {

enum Epi { EPI_F32 = 0, EPI_BF16, EPI_ADD_F32, EPI_SWIGLU_BF16, EPI_SWIGLU_F32, EPI_LMHEAD };

constexpr int BKB = 128;             // K bytes per stage row

// A k-group is WM x WN = 4 or 8 waves, each owning a (BM / WM) x (BN / WN)
// block of the tile.  KW_ k-groups share the tile and the LDS ring; k-group g
// computes k-steps g, g + KW, ... of every stage, and the groups' accumulators
// are added through LDS before the epilogue.  Two k-groups (or an 8-wave
// group) put two waves on each SIMD, which doubles the LDS fragment bandwidth
// a SIMD can draw (one wave reads at most ~27 B per clock from LDS).
template <typename T, int BM_, int BN_, int WM_, int WN_, bool DUAL, int NS, int KW_ = 1>
struct Core {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr bool TWO_B = DUAL;
    static constexpr int TM = BM / WM / 16;
    static constexpr int TN = BN / WN / 16;
    static constexpr int KSB = Mfma<T>::KSTEP * (int)sizeof(T);   // K bytes per step
    static constexpr int LB = Mfma<T>::LANE_BYTES;
    static constexpr int ROWS = BM + BN * (DUAL ? 2 : 1);           // rows per stage
    static constexpr int STAGE = ROWS * BKB;
    static constexpr int LDS_BYTES = NS * STAGE;
    static constexpr int KW = KW_;
    static constexpr int NPOS = WM * WN;                            // waves per k-group
    static constexpr int NWAVES = NPOS * KW;
    static constexpr int THREADS = WAVE * NWAVES;
    static constexpr int LPW = ROWS / 8 / NWAVES;                   // 1-KB loads per wave per stage
    static constexpr int KS = BKB / KSB;                            // MFMA k-steps per stage
    static constexpr int KSW = KS / KW;                             // ... per k-group
    static constexpr int PART = TM * TN * 4;
    typedef typename Mfma<T>::frag frag;
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile");
    static_assert(NPOS == 4 || NPOS == 8, "4 or 8 waves per k-group");
    static_assert(ROWS % (8 * NWAVES) == 0 && KS % KW == 0, "stage rows / k-steps");
    static_assert((NS - 2) * LPW < 64, "vmcnt");

    const uint8_t* src[LPW];     // this lane's source (row + swizzled chunk) per load
    int kstep[LPW];              // bytes from one K stage to the next for that load
    f32x4 acc[TM][TN];
    f32x4 acc2[DUAL ? TM : 1][DUAL ? TN : 1];
    int wave;                    // 0 .. NWAVES - 1
    int pos;                     // wave within the k-group: (wm, wn) = (pos / WN, pos % WN)
    int kg;                      // k-group

    // rowptr(R, step) -> address of stage row R's first K stage (A rows, then
    // B, then B2) and, in step, the bytes to its next stage; always a readable
    // row (rows outside the matrix are clamped by the caller: they only feed
    // outputs that are not stored).  A load instruction covers 8 rows, all of A
    // or all of one B (BM and BN are multiples of 8), so its step is uniform.
    template <class F>
    __device__ __forceinline__ void init(F rowptr) {
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
        pos = wave % NPOS;
        kg = wave / NPOS;
        const int lane = threadIdx.x % WAVE;
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int R = (wave * LPW + j) * 8 + lane / 8;
            const int chunk = (lane % 8) ^ (R & 7);
            int step = BKB;
            src[j] = rowptr(R, step) + chunk * 16;
            kstep[j] = __builtin_amdgcn_readfirstlane(step);
        }
    }

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (DUAL) acc2[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
    }

    __device__ __forceinline__ void load_stage(uint8_t* smem, int kt, int slot) {
        uint8_t* dst = smem + slot * STAGE + wave * LPW * 1024;
#pragma unroll
        for (int j = 0; j < LPW; ++j)
            __builtin_amdgcn_global_load_lds((const void*)(src[j] + (long)kt * kstep[j]), (lds_ptr)(dst + j * 1024), 16,
                                             0, 0);
    }

    // Fragments of one stage as read from LDS (fp8 codes are widened at use).
    typedef typename Mfma<T>::raw raw;
    struct Frags {
        raw a[KSW][TM], b[KSW][TN], b2[KSW][DUAL ? TN : 1];
    };
    // Register double-buffering of fragments when both sets, their widened
    // copies (fp8) and the accumulators fit a wave's registers (512 with one
    // wave per SIMD, 256 with two).
    static constexpr int FRAG_REGS = KSW * (TM + TN * (DUAL ? 2 : 1)) * 4;
    static constexpr int ACC_REGS = TM * TN * 4 * (DUAL ? 2 : 1);
    static constexpr bool DB =
        2 * FRAG_REGS + (sizeof(T) == 1 ? 2 * FRAG_REGS : 0) + ACC_REGS <= (NWAVES == 4 ? 400 : 190);
    static_assert(KW == 1 || WAVE * NPOS * ACC_REGS * 4 <= LDS_BYTES, "k-group exchange fits the LDS ring");

    __device__ __forceinline__ void read(Frags& f, const uint8_t* stage) const {
        const int lane = threadIdx.x % WAVE;
        const int wm = pos / WN, wn = pos % WN;
        const int sw = lane & 7;                       // rows of a fragment are 16-aligned: row & 7 == lane & 7
        const uint8_t* sa = stage + (wm * (BM / WM) + lane % 16) * BKB;
        const uint8_t* sb = stage + (BM + wn * (BN / WN) + lane % 16) * BKB;
#pragma unroll
        for (int ss = 0; ss < KSW; ++ss) {
            const int off = (ss * KW + kg) * KSB + (lane / 16) * LB;
            const int phys = (((off >> 4) ^ sw) << 4) | (off & 15);
#pragma unroll
            for (int i = 0; i < TM; ++i) f.a[ss][i] = Mfma<T>::load(sa + i * 16 * BKB + phys);
#pragma unroll
            for (int j = 0; j < TN; ++j) f.b[ss][j] = Mfma<T>::load(sb + j * 16 * BKB + phys);
            if constexpr (DUAL) {
#pragma unroll
                for (int j = 0; j < TN; ++j) f.b2[ss][j] = Mfma<T>::load(sb + (BN + j * 16) * BKB + phys);
            }
        }
    }

    __device__ __forceinline__ void mma(const Frags& f) {
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            frag af[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i] = Mfma<T>::widen(f.a[s][i]);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const frag bf = Mfma<T>::widen(f.b[s][j]);
#pragma unroll
                for (int i = 0; i < TM; ++i) acc[i][j] = Mfma<T>::mac(af[i], bf, acc[i][j]);
            }
            if constexpr (DUAL) {
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const frag bf = Mfma<T>::widen(f.b2[s][j]);
#pragma unroll
                    for (int i = 0; i < TM; ++i) acc2[i][j] = Mfma<T>::mac(af[i], bf, acc2[i][j]);
                }
            }
        }
    }

    // Accumulates K stages [kt0, kt1).  Fragments are double-buffered in
    // registers: after stage t+1's barrier its fragment reads are issued, then
    // stage t's MFMAs (from the other register set), so LDS latency hides
    // under the MFMAs; the slot of stage t (already in registers everywhere)
    // is refilled with stage t + NS.
    __device__ __forceinline__ void run(uint8_t* smem, int kt0, int kt1) {
        zero();
        const int n = kt1 - kt0;
        if (n <= 0) return;
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < n) load_stage(smem, kt0 + s, s);
        if constexpr (!DB) {
            Frags f;
            for (int t = 0; t < n; ++t) {
                wait_stages<LPW, NS - 2>(min(NS - 2, n - 1 - t));
                stage_barrier();
                if (t + NS - 1 < n) load_stage(smem, kt0 + t + NS - 1, (t + NS - 1) % NS);
                read(f, smem + (t % NS) * STAGE);
                mma(f);
                constexpr int NREAD = KSW * (TM + TN * (DUAL ? 2 : 1));
                constexpr int NMFMA = KSW * TM * TN * (DUAL ? 2 : 1) * (sizeof(T) == 1 ? 2 : 1);
                __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);
            }
            return;
        }
        Frags f0, f1;
        wait_stages<LPW, NS - 2>(min(NS - 2, n - 1));
        stage_barrier();
        read(f0, smem);
        if (NS - 1 < n) load_stage(smem, kt0 + NS - 1, NS - 1);
        // one stage: stage t is in `cur`; stage t + 1 (< n) is read into `nxt`
        auto step = [&](int t, Frags& cur, Frags& nxt) {
            wait_stages<LPW, NS - 2>(min(NS - 2, n - 2 - t));
            stage_barrier();
            if (t + NS < n) load_stage(smem, kt0 + t + NS, (t + NS) % NS);
            read(nxt, smem + ((t + 1) % NS) * STAGE);
            mma(cur);
            // keep the reads as one group ahead of the MFMAs through scheduling
            constexpr int NREAD = KSW * (TM + TN * (DUAL ? 2 : 1));
            constexpr int NMFMA = KSW * TM * TN * (DUAL ? 2 : 1) * (sizeof(T) == 1 ? 2 : 1);
            __builtin_amdgcn_sched_group_barrier(0x100, NREAD, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, NMFMA, 0);
        };
        int t = 0;
        for (; t + 2 < n; t += 2) {
            step(t, f0, f1);
            step(t + 1, f1, f0);
        }
        if (t + 1 < n) {
            step(t, f0, f1);
            mma(f1);
        } else {
            mma(f0);
        }
    }

    // Adds every k-group's accumulators into k-group 0 through LDS (the ring is
    // free: run() ended with all loads waited for); true for the waves that
    // then hold the tile's result.  Fixed order: group 0 + group 1.
    __device__ __forceinline__ bool reduce(uint8_t* smem) {
        if constexpr (KW == 1) {
            return true;
        } else {
            const int lane = threadIdx.x % WAVE;
            float* x = (float*)smem + (long)pos * ACC_REGS * WAVE + lane;   // [pos][reg][lane]
            __syncthreads();
            if (kg == 1) {
                int r = 0;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            x[(r++) * WAVE] = acc[i][j][v];
                            if constexpr (DUAL) x[(r++) * WAVE] = acc2[i][j][v];
                        }
            }
            __syncthreads();
            if (kg == 0) {
                int r = 0;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            acc[i][j][v] += x[(r++) * WAVE];
                            if constexpr (DUAL) acc2[i][j][v] += x[(r++) * WAVE];
                        }
            }
            return kg == 0;
        }
    }
};

// Weight rows in the tiled layout: blocks of TILE_ROWS rows x BKB bytes, so a
// K stage of TILE_ROWS consecutive rows is one contiguous 2 KB run (DRAM pages
// are read whole instead of one 128-byte line per row); block (g, kt) of a
// matrix with nkt stages per row starts at byte (g * nkt + kt) * TILE_BYTES.
constexpr int TILE_ROWS = 16;
constexpr int TILE_BYTES = TILE_ROWS * BKB;

// Address of weight row r's first K stage and the step to its next stage.
__device__ __forceinline__ const uint8_t* brow(const uint8_t* B, long ldb, bool tiled, int nkt, int r, int& step) {
    if (!tiled) {
        step = BKB;
        return B + (long)r * ldb;
    }
    step = TILE_BYTES;
    return B + ((long)(r / TILE_ROWS) * nkt) * TILE_BYTES + (r % TILE_ROWS) * BKB;
}

// Remap a linear workgroup id so each XCD (id % 8) gets a contiguous range.
__device__ __forceinline__ int xcd_remap(int b, int total) {
    if (total % 8 != 0) return b;
    return (b % 8) * (total / 8) + b / 8;
}

struct EpiArgs {
    void* C; long ldc;                   // elements
    const float* a_scale;                // fp8: per A-source-row
    const float* b_scale;                // fp8: per output column
    const float* b2_scale;
    // LM head
    float* pmax; float* psum; int* pidx; int n_tiles; int mask_col;
    float* logits; long ld_logits;
};

// One output element: x = accumulated A B^T (u: the second weight's, SwiGLU).
template <int EPI, bool FP8>
__device__ __forceinline__ void epi_elem(const EpiArgs& e, int row, int col, int src_row, float x, float u) {
    if constexpr (FP8) {
        const float sa = e.a_scale[src_row];
        x *= sa * e.b_scale[col];
        if constexpr (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_F32) u *= sa * e.b2_scale[col];
    }
    const long off = (long)row * e.ldc + col;
    if constexpr (EPI == EPI_F32) {
        ((float*)e.C)[off] = x;
    } else if constexpr (EPI == EPI_BF16) {
        ((bf16_t*)e.C)[off] = f32_to_bf16(x);
    } else if constexpr (EPI == EPI_ADD_F32) {
        ((float*)e.C)[off] += x;
    } else if constexpr (EPI == EPI_SWIGLU_BF16) {
        ((bf16_t*)e.C)[off] = f32_to_bf16(silu_f(x) * u);
    } else if constexpr (EPI == EPI_SWIGLU_F32) {
        ((float*)e.C)[off] = silu_f(x) * u;
    }
}

// Applies the epilogue to one wave's accumulators.
template <class C, bool FP8, int EPI>
__device__ __forceinline__ void epilogue(C& c, const EpiArgs& e, int m0, int n0, int mlim, int N, const int* gather,
                                         int gather_div, int ntile) {
    const int lane = threadIdx.x % WAVE;
    const int wm = c.pos / C::WN, wn = c.pos % C::WN;
    const int rbase = m0 + wm * (C::BM / C::WM) + 4 * (lane / 16);
    const int cbase = n0 + wn * (C::BN / C::WN) + lane % 16;
    if constexpr (EPI == EPI_LMHEAD) {
        // one partial per (row, column slice of a wave): slice ntile * WN + wn
        // of width BN / WN; a slice wholly past N (a ragged last tile) has
        // none
        const int slice = ntile * C::WN + wn;
        const bool sok = slice < e.n_tiles;
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = rbase + i * 16 + v;
                const bool rok = row < mlim;
                float sa = 1.f;
                if constexpr (FP8) sa = rok ? e.a_scale[row] : 1.f;
                float vals[C::TN];
                float mx = -INFINITY;
                int ix = 0x7fffffff;
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const int col = cbase + j * 16;
                    float x = c.acc[i][j][v];
                    if constexpr (FP8) x *= sa * (col < N ? e.b_scale[col] : 0.f);
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
                if (rok && sok && lane % 16 == 0) {
                    const long k = (long)row * e.n_tiles + slice;
                    e.pmax[k] = mx;
                    e.psum[k] = s;
                    e.pidx[k] = ix;
                }
            }
    } else {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = rbase + i * 16 + v;
                if (row >= mlim) continue;
                const int src = gather ? gather[row] / gather_div : row;
#pragma unroll
                for (int j = 0; j < C::TN; ++j) {
                    const int col = cbase + j * 16;
                    if (col >= N) continue;
                    float u = 0.f;
                    if constexpr (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_F32) u = c.acc2[i][j][v];
                    epi_elem<EPI, FP8>(e, row, col, src, c.acc[i][j][v], u);
                }
            }
    }
}

// Raw split-K partials: part[split][row][col] (and the second weight's at
// part2) for rows < M, cols < N.
template <class C>
__device__ __forceinline__ void store_partial(C& c, float* part, float* part2, int m0, int n0, int M, int N) {
    const int lane = threadIdx.x % WAVE;
    const int wm = c.pos / C::WN, wn = c.pos % C::WN;
    const int rbase = m0 + wm * (C::BM / C::WM) + 4 * (lane / 16);
    const int cbase = n0 + wn * (C::BN / C::WN) + lane % 16;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = rbase + i * 16 + v;
            if (row >= M) continue;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int col = cbase + j * 16;
                if (col >= N) continue;
                part[(long)row * N + col] = c.acc[i][j][v];
                if constexpr (C::TWO_B) part2[(long)row * N + col] = c.acc2[i][j][v];
            }
        }
}

struct DenseArgs {
    const uint8_t* A; long lda;          // bytes
    const uint8_t* B; const uint8_t* B2; long ldb;
    int b_tiled;                         // B / B2 in the tiled layout (ldb unused)
    int M, N, K;
    int splits;                          // split-K factor (1 = none)
    float* part;                         // [splits][M][N] (+ the same again for the second weight)
    EpiArgs e;
};

// Workgroup order: ((n-tile * splits + split) * m-tiles + m-tile), remapped so
// each XCD runs a contiguous range of it.
template <class C, typename T, int EPI>
__global__ __launch_bounds__(C::THREADS) void gemm_dense_kernel(DenseArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];
    const int mt_n = (a.M + C::BM - 1) / C::BM, nt_n = (a.N + C::BN - 1) / C::BN;
    const int lin = xcd_remap(blockIdx.x, mt_n * nt_n * a.splits);
    const int mt = lin % mt_n;
    const int split = (lin / mt_n) % a.splits;
    const int nt = lin / mt_n / a.splits;
    const int m0 = mt * C::BM, n0 = nt * C::BN;
    const int nkt = (int)((long)a.K * sizeof(T) / BKB);
    C c;
    c.init([&](int R, int& step) -> const uint8_t* {
        if (R < C::BM) {
            const int r = min(m0 + R, a.M - 1);
            return a.A + (long)r * a.lda;
        }
        R -= C::BM;
        const uint8_t* B = a.B;
        if (R >= C::BN) { R -= C::BN; B = a.B2; }
        return brow(B, a.ldb, a.b_tiled, nkt, min(n0 + R, a.N - 1), step);
    });
    const int per = (nkt + a.splits - 1) / a.splits;
    c.run(smem, split * per, min(nkt, (split + 1) * per));
    if (!c.reduce(smem)) return;
    if (a.splits > 1) {
        const long mn = (long)a.M * a.N;
        store_partial(c, a.part + split * mn, a.part + (a.splits + split) * mn, m0, n0, a.M, a.N);
        return;
    }
    epilogue<C, sizeof(T) == 1, EPI>(c, a.e, m0, n0, a.M, a.N, nullptr, 1, nt);
}

// Sum of the split partials in split order, then the epilogue.
template <int EPI, bool FP8, bool DUAL>
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(const float* part, int splits, int M, int N,
                                                               EpiArgs e) {
    const int row = blockIdx.y;
    const int col = blockIdx.x * 256 + threadIdx.x;
    if (col >= N) return;
    const long mn = (long)M * N, off = (long)row * N + col;
    float x = 0.f, u = 0.f;
    for (int s = 0; s < splits; ++s) {
        x += part[s * mn + off];
        if constexpr (DUAL) u += part[(splits + s) * mn + off];
    }
    epi_elem<EPI, FP8>(e, row, col, row, x, u);
}

struct GroupedArgs {
    const uint8_t* A; long lda;          // bytes
    const int* gather; int gather_div;   // A row of permuted row p = gather[p] / gather_div (nullable)
    const uint8_t* B; const uint8_t* B2; long ldb; long b_stride;   // bytes between experts
    int b_tiled;
    const float* b_scale; const float* b2_scale; long bs_stride;     // elements between experts
    const int* offs;        // [E + 1] permuted row offsets per expert
    const int* tile_start;  // [E + 1] first m-tile of each expert (for this BM)
    int E, max_mtiles, N, K;
    EpiArgs e;
};

template <class C, typename T, int EPI>
__global__ __launch_bounds__(C::THREADS) void gemm_grouped_kernel(GroupedArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[C::LDS_BYTES];
    // Only the first mtiles = tile_start[E] m-tiles exist (the grid is sized
    // for the most there can be).  The mtiles * nt_n live tiles are dealt to the 8 XCDs
    // (blockIdx % 8) in equal contiguous ranges, so each XCD streams the same
    // share of expert weights; inside a range the m-tiles of one weight tile
    // are adjacent and share that XCD's L2.
    const int nt_n = (a.N + C::BN - 1) / C::BN;
    const int mtiles = a.tile_start[a.E];
    const int live = mtiles * nt_n;
    const int per = (live + 7) / 8;
    const int slot = blockIdx.x / 8;
    if (slot >= per) return;
    const int lin = (blockIdx.x % 8) * per + slot;
    if (lin >= live) return;
    const int nt = lin / mtiles, mt = lin % mtiles;
    // expert owning m-tile mt: last e with tile_start[e] <= mt
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int ex = lo;
    const int m0 = a.offs[ex] + (mt - a.tile_start[ex]) * C::BM;
    const int mlim = a.offs[ex + 1];
    const int n0 = nt * C::BN;
    const uint8_t* Be = a.B + (long)ex * a.b_stride;
    const uint8_t* B2e = C::TWO_B ? a.B2 + (long)ex * a.b_stride : nullptr;
    const int nkt = (int)((long)a.K * sizeof(T) / BKB);
    C c;
    c.init([&](int R, int& step) -> const uint8_t* {
        if (R < C::BM) {
            const int r = min(m0 + R, mlim - 1);
            const int src = a.gather ? a.gather[r] / a.gather_div : r;
            return a.A + (long)src * a.lda;
        }
        R -= C::BM;
        const uint8_t* B = Be;
        if (R >= C::BN) { R -= C::BN; B = B2e; }
        return brow(B, a.ldb, a.b_tiled, nkt, min(n0 + R, a.N - 1), step);
    });
    c.run(smem, 0, nkt);
    if (!c.reduce(smem)) return;
    EpiArgs e = a.e;
    if constexpr (sizeof(T) == 1) {
        e.b_scale = a.b_scale + (long)ex * a.bs_stride;
        if (a.b2_scale) e.b2_scale = a.b2_scale + (long)ex * a.bs_stride;
    }
    epilogue<C, sizeof(T) == 1, EPI>(c, e, m0, n0, mlim, a.N, a.gather, a.gather_div, nt);
}

// ------------------------------------------------------------- launchers --

// Tile shapes (BM, BN, WM, WN, stages):
//   small M (<= 64; the tiny model, short canvases)     32 x 64,  waves 1x4, 4 stages
//   canvas M (<= 256; one request's canvas)             64 x 64,  waves 2x2 x 2 k-groups, 6 stages
//     (SwiGLU pair: 128 x 64 x 2 weights, 2 k-groups, if N >= 4096, else 64 x 32 x 2)
//   prefill M                                           128 x 128, waves 2x2 x 2 k-groups, 4 stages; SwiGLU pair
//                                                       256 x 128 x 2, waves 4x2, 2 stages (fp8: 128 x 128 x 2, 2 k-groups);
//                                                       single weight: 256 x 256, waves 4x2, 2 stages (fp8: 128 x 256)
//                                                       when 128 x 256 tiles number >= 256,
//                                                       128 x 64 for a short-K residual add that 128 x 128 leaves the chip idle
//   LM head (one partial per wave column slice)         64 x 64 (waves 4x1) / 256 x 256 (waves 4x2; fp8: 256 x 128, 4x1 x 2 k-groups)
//   grouped (experts)                                   SwiGLU pair 64 x 64 x 2, else 64 x 128; waves 2x2, 3 stages
//                                                       (fp8: 2 k-groups); >= 256 rows per expert on average:
//                                                       SwiGLU pair 128 x 128 (2 k-groups), else 128 x 256 (waves 2x4);
//                                                       bf16, >= 512 rows per expert: 256 x 128 x 2 / 256 x 256 (waves 4x2)
//                                                       (BM = grouped_bm)
// The canvas choices come from a sweep of every variant and split factor on
// the workloads' projection shapes: small tiles give enough workgroups to keep
// weight bytes in flight on every CU; the m-tiles sharing a weight tile are
// adjacent in the XCD-aware order, so the weights are fetched from HBM once.
// The wider LM-head tile halves the activation re-reads over the vocabulary.
template <typename T, bool DUAL> using CoreS = Core<T, 32, 64, 1, 4, DUAL, 4>;
template <typename T, bool DUAL> using CoreM = Core<T, 64, 64, 2, 2, DUAL, 4>;
template <typename T, bool DUAL>
using CoreW = std::conditional_t<DUAL, Core<T, 128, 64, 2, 2, true, 4>, Core<T, 256, 64, 4, 1, false, 3>>;
// Prefill SwiGLU pair: 256 x 128 x 2 weights over 8 waves of 64 x 64 x 2
// (one k-group, 2 stages) -- twice the rows per weight tile of 128 x 128;
// measured on the 32-request MoE step (8192 canvas rows): shared expert's
// gate/up 7.8 -> 5.9 ms per step.  fp8 keeps 128 x 128 x 2 with two k-groups
// (its widened fragments spill at 256 rows).
template <typename T, bool DUAL>
using CoreL = std::conditional_t<DUAL && sizeof(T) != 1, Core<T, 256, 128, 4, 2, true, 2, 1>,
                                 Core<T, 128, 128, 2, 2, DUAL, DUAL ? 3 : 4, 2>>;
// Wide single-weight tile (fp8 prefill-sized M): each wave's 64 x 128 block
// reads 12 fragments per 32 MFMAs instead of 8 per 16 (a 128 x 128 tile's
// 64 x 64 blocks).
template <typename T> using CoreLW = Core<T, 128, 256, 2, 2, false, 3, 2>;
// Dense prefill single-weight tile: 256 x 256 over 8 waves of 64 x 128, one
// k-group and 2 stages (twice the rows per weight tile of CoreLW; shared
// expert's down projection on the 32-request step: 11.6 -> 8.7 ms).  fp8
// stays on CoreLW: its widened fragments spill at 256 x 256.
template <typename T>
using CoreLD = std::conditional_t<sizeof(T) == 1, CoreLW<T>, Core<T, 256, 256, 4, 2, false, 2, 1>>;
template <typename T> using CoreHs = Core<T, 64, 64, 4, 1, false, 4>;
// LM head at canvas M: a 256 x 256 tile of 8 waves (64 x 128 each), two
// stages -- each activation K-slice in LDS feeds twice the vocabulary of a
// 256 x 128 tile (measured on the 256 x 262144 x 2560 head: 438-452 us ->
// 345-349).  fp8 keeps 256 x 128 with two k-groups (its widened fragments
// would spill at 256 x 256).
template <typename T>
using CoreHw = std::conditional_t<sizeof(T) == 1, Core<T, 256, 128, 4, 1, false, 3, 2>,
                                  Core<T, 256, 256, 4, 2, false, 2, 1>>;
// Expert tiles: 64 rows (about what one expert gets from a 256-row canvas at
// top-8 of 128) and 3 stages, from a sweep over routings that touch 32 to 69
// experts; wider weight tiles for the narrow-K down projection.  fp8 tiles run
// two k-groups: a 128-byte stage holds twice the products of a bf16 one, and
// the extra waves hide the E4M3 widening (measured 6% faster; bf16 0.4% slower).
template <typename T, bool DUAL>
using CoreG = std::conditional_t<sizeof(T) == 1,
                                 std::conditional_t<DUAL, Core<T, 64, 64, 2, 2, true, 3, 2>, Core<T, 64, 128, 2, 2, false, 3, 2>>,
                                 std::conditional_t<DUAL, Core<T, 64, 64, 2, 2, true, 3>, Core<T, 64, 128, 2, 2, false, 3>>>;
// Experts that average 256 rows or more (many requests' canvases, prompts)
// are compute-bound: 128-row tiles, 128 x 128 with two k-groups for the
// SwiGLU pair (wider pair tiles measured slower: more padding rows' work per
// ragged expert; so did 8 waves of 64 x 32 x 2) and, for the down
// projection, 128 x 256 over 8 waves of 64 x 64 with one k-group (expert
// down on the 32-request step: 15.7 -> 14.0 ms against the 4-wave wide tile).
template <typename T, bool DUAL>
using CoreGL = std::conditional_t<DUAL, Core<T, 128, 128, 2, 2, true, 3, 2>, Core<T, 128, 256, 2, 4, false, 3, 1>>;
// bf16 experts averaging 512 rows or more (the 32-request step: 65536
// assignments over 128 experts) take 256-row m-tiles over 8 wave positions:
// 256 x 128 x 2 for the SwiGLU pair, 256 x 256 for the down projection (one
// k-group, 2 stages) -- twice the rows per weight tile outweighs the longer
// padding of ragged experts there: expert gate/up 22.0 -> 20.1 ms, down 13.6
// -> 12.4 ms per step.  At ~256 rows per expert (a 4096-token prompt) the
// padding would cost more than it saves.
template <typename T, bool DUAL>
using CoreGX = std::conditional_t<DUAL, Core<T, 256, 128, 4, 2, true, 2, 1>, Core<T, 256, 256, 4, 2, false, 2, 1>>;
static_assert(CoreG<float, true>::BM == CoreG<float, false>::BM && CoreG<bf16_t, true>::BM == CoreG<bf16_t, false>::BM &&
              CoreG<fp8_t, true>::BM == CoreG<fp8_t, false>::BM && CoreGL<bf16_t, true>::BM == CoreGL<bf16_t, false>::BM &&
              CoreGL<fp8_t, true>::BM == CoreGL<bf16_t, true>::BM && CoreGL<float, true>::BM == CoreGL<bf16_t, true>::BM &&
              CoreGX<bf16_t, true>::BM == CoreGX<bf16_t, false>::BM,
              "one expert m-tile height per operand type and tile family");

static bool grouped_large(int n_assign, int E) { return (long)n_assign >= 256L * E; }
static bool grouped_huge(int dtype, int n_assign, int E) { return dtype == DT_BF16 && (long)n_assign >= 512L * E; }

bool grouped_compute_bound(int n_assign, int E) { return grouped_large(n_assign, E); }

int grouped_bm(int dtype, int n_assign, int E) {
    if (grouped_huge(dtype, n_assign, E)) return CoreGX<bf16_t, true>::BM;
    if (grouped_large(n_assign, E)) return CoreGL<bf16_t, true>::BM;
    switch (dtype) {
        case DT_F32: return CoreG<float, true>::BM;
        case DT_FP8: return CoreG<fp8_t, true>::BM;
        default: return CoreG<bf16_t, true>::BM;
    }
}

constexpr int SPLIT_TARGET_WG = 256;

// Split-K factor: enough workgroups for the chip when the output tiles alone
// are too few; every split keeps at least 4 K-stages; equalised so that no
// split is empty.  LM-head GEMMs are never split; prefill-sized ones only as a
// residual add with a long K and too few tiles (in two).
template <class C, typename T, int EPI>
static int splits_for(const GemmDesc& d) {
    if constexpr (EPI == EPI_LMHEAD) return 1;
    const long tiles = (long)((d.M + C::BM - 1) / C::BM) * ((d.N + C::BN - 1) / C::BN);
    const int nkt = (int)((long)d.K * sizeof(T) / BKB);
    if (d.force_splits > 0) {
        const int per = (nkt + std::min(d.force_splits, nkt) - 1) / std::min(d.force_splits, nkt);
        return (nkt + per - 1) / per;
    }
    // a SwiGLU split would need its own epilogue kernel (the nonlinearity
    // needs the full sums): never split it
    // tiles of two k-groups already put 8 waves on a CU: splitting a plain
    // store measured slower from 160 tiles up; a residual add still gains
    // (split partials are plain stores summed by the next kernel, where the
    // unsplit epilogue reads and rewrites the fp32 stream)
    if (d.M > 256) {
        // prefill-sized: only a residual add with a long K and too few tiles
        // for the chip splits, in two (the dense FFN's down projection at a
        // 1024-token prompt: 42 us against 80 unsplit on 128 x 128 tiles)
        if (C::TWO_B || EPI != EPI_ADD_F32 || tiles >= SPLIT_TARGET_WG || d.K < 4L * d.N || nkt < 8) return 1;
        const int per = (nkt + 1) / 2;
        return (nkt + per - 1) / per;
    }
    const long no_split = (C::KW > 1 && EPI != EPI_ADD_F32) ? 160 : SPLIT_TARGET_WG * 3 / 4;
    if (C::TWO_B || tiles >= no_split) return 1;
    int s = (int)((SPLIT_TARGET_WG + tiles - 1) / tiles);
    s = std::min(s, std::max(1, nkt / 4));
    s = std::min(s, 2);
    const int per = (nkt + s - 1) / s;
    return std::max(1, (nkt + per - 1) / per);
}

template <class C, typename T, bool DUAL, int EPI>
static long part_floats(const GemmDesc& d) {
    const int s = splits_for<C, T, EPI>(d);
    return s == 1 ? 0 : (long)s * d.M * d.N * (DUAL ? 2 : 1);
}

// bn: the columns one LM-head partial covers (BN / WN of the tile)
static EpiArgs make_epi(const GemmDesc& d, int bn) {
    EpiArgs e;
    e.C = d.C; e.ldc = d.ldc;
    e.a_scale = d.a_scale; e.b_scale = d.b_scale; e.b2_scale = d.b2_scale;
    e.pmax = d.pmax; e.psum = d.psum; e.pidx = d.pidx; e.n_tiles = (d.N + bn - 1) / bn;
    e.mask_col = d.mask_col; e.logits = d.logits; e.ld_logits = d.ld_logits;
    return e;
}

// Launches the GEMM; returns its split-K factor.
template <class C, typename T, bool DUAL, int EPI>
static int launch_dense(const GemmDesc& d, hipStream_t st) {
    DenseArgs a;
    a.A = (const uint8_t*)d.A; a.lda = d.lda * (long)sizeof(T);
    a.B = (const uint8_t*)d.B; a.B2 = (const uint8_t*)d.B2; a.ldb = d.ldb * (long)sizeof(T);
    a.b_tiled = d.b_tiled ? 1 : 0;
    a.M = d.M; a.N = d.N; a.K = d.K;
    a.splits = splits_for<C, T, EPI>(d);
    if (a.splits > 1 && (!d.splitk || part_floats<C, T, DUAL, EPI>(d) > d.splitk_floats))
        a.splits = 1;   // no room: unsplit (correct, fewer workgroups)
    a.part = d.splitk;
    a.e = make_epi(d, C::BN / C::WN);
    const int grid = ((d.M + C::BM - 1) / C::BM) * ((d.N + C::BN - 1) / C::BN) * a.splits;
    if (grid == 0) return 1;
    launch((gemm_dense_kernel<C, T, EPI>), dim3(grid), dim3(C::THREADS), 0, st, a);
    return a.splits;
}

template <typename T, bool DUAL, int EPI>
static void finish_dense(const GemmDesc& d, int splits, hipStream_t st) {
    if constexpr (EPI != EPI_LMHEAD) {
        const EpiArgs e = make_epi(d, 64);
        launch((splitk_epilogue_kernel<EPI, sizeof(T) == 1, DUAL>), dim3((d.N + 255) / 256, d.M),
                           dim3(256), 0, st, d.splitk, splits, d.M, d.N, e);
    }
}

template <class C, typename T, int EPI>
static void launch_grouped(const GemmDesc& d, hipStream_t st) {
    GroupedArgs a;
    a.A = (const uint8_t*)d.A; a.lda = d.lda * (long)sizeof(T);
    a.gather = d.gather; a.gather_div = d.gather_div;
    a.B = (const uint8_t*)d.B; a.B2 = (const uint8_t*)d.B2; a.ldb = d.ldb * (long)sizeof(T);
    a.b_tiled = d.b_tiled ? 1 : 0;
    a.b_stride = d.b_stride * (long)sizeof(T);
    a.b_scale = d.b_scale; a.b2_scale = d.b2_scale; a.bs_stride = d.bs_stride;
    a.offs = d.offs; a.tile_start = d.tile_start; a.E = d.E; a.N = d.N; a.K = d.K;
    a.max_mtiles = (d.M + C::BM - 1) / C::BM + d.E;
    a.e = make_epi(d, C::BN);
    // a multiple of 8 covers the 8 equal XCD ranges of any live tile count
    const int grid = (a.max_mtiles * ((d.N + C::BN - 1) / C::BN) + 7) / 8 * 8;
    if (d.M == 0 || grid == 0) return;
    launch((gemm_grouped_kernel<C, T, EPI>), dim3(grid), dim3(C::THREADS), 0, st, a);
}

// Tile variants a caller may force (GemmDesc::variant, the GEMM test entry
// point): bf16 operands, fp32-store or SwiGLU epilogue.
template <typename T, bool DUAL, class F>
static bool with_variant(int v, F f) {
    switch (v) {
        case 1: f(Core<T, 128, 64, 2, 2, DUAL, 4>{}); return true;
        case 2: f(Core<T, 64, 64, 2, 2, DUAL, 4>{}); return true;
        case 3: f(Core<T, 256, 64, 4, 1, DUAL, 3>{}); return true;
        case 4: f(Core<T, 128, 128, 2, 2, DUAL, DUAL ? 3 : 4>{}); return true;
        case 5: f(Core<T, 64, 128, 2, 2, DUAL, DUAL ? 3 : 4>{}); return true;
        case 6: f(Core<T, 64, 32, 2, 2, DUAL, 4>{}); return true;
        case 7: f(Core<T, 32, 64, 1, 4, DUAL, 4>{}); return true;
        case 8: f(Core<T, 64, 64, 2, 2, DUAL, 6>{}); return true;
        case 9: f(Core<T, 128, 64, 2, 2, DUAL, 4, 2>{}); return true;
        case 10: f(Core<T, 64, 64, 2, 2, DUAL, 4, 2>{}); return true;
        case 11: f(Core<T, 128, 128, 2, 2, DUAL, DUAL ? 3 : 4, 2>{}); return true;
        case 12: f(Core<T, 64, DUAL ? 32 : 64, 2, 2, DUAL, DUAL ? 4 : 6, 2>{}); return true;
        default: return false;
    }
}
constexpr int GEMM_VARIANTS = 12;

template <bool DUAL, int EPI, typename T, class F>
static void with_core(const GemmDesc& d, F f) {
    if constexpr (std::is_same_v<T, bf16_t> && (EPI == EPI_F32 || EPI == EPI_SWIGLU_BF16)) {
        if (d.variant && with_variant<T, DUAL>(d.variant, f)) return;
    }
    if constexpr (EPI == EPI_LMHEAD) {
        if (d.M <= 64) f(CoreHs<T>{});
        else f(CoreHw<T>{});
    } else {
        if (d.M <= 64) f(CoreS<T, DUAL>{});
        else if (d.M <= 256) {
            // measured on the canvas shapes (M = 256) with weights streamed
            // from HBM: 64 x 64 tiles, 6 stages, two k-groups for the
            // projections; a SwiGLU pair gets 128 x 64 tiles with two k-groups
            // when wide, 64 x 32 when narrow
            if constexpr (DUAL) {
                if (d.N >= 4096) f(Core<T, 128, 64, 2, 2, true, 4, 2>{});
                else f(Core<T, 64, 32, 2, 2, true, 4>{});
            } else {
                f(Core<T, 64, 64, 2, 2, false, 6, 2>{});
            }
        } else {
            // prefill-sized M: 128 x 128 tiles with two k-groups (SwiGLU
            // pair: 256 x 128 x 2), or the 256 x 256 tile when 128 x 256
            // tiles would still give a workgroup per CU; a
            // residual add whose 128 x 128 tiles would leave CUs idle and
            // whose K is short (the O projection at a 1024-token prompt: 16.4
            // us against 24.5) takes 128 x 64 tiles instead
            const long t128 = (long)((d.M + 127) / 128) * ((d.N + 127) / 128);
            if constexpr (!DUAL) {
                if ((long)((d.M + 127) / 128) * ((d.N + 255) / 256) >= SPLIT_TARGET_WG) {
                    f(CoreLD<T>{});
                    return;
                }
            }
            if constexpr (!DUAL && EPI == EPI_ADD_F32) {
                if (t128 < SPLIT_TARGET_WG && d.K < 4L * d.N) {
                    f(Core<T, 128, 64, 2, 2, false, 4, 2>{});
                    return;
                }
            }
            f(CoreL<T, DUAL>{});
        }
    }
}

enum DenseOp { OP_LAUNCH, OP_NEED, OP_FINISH };

// OP_LAUNCH: launch, *io = splits.  OP_NEED: *io = partial floats.
// OP_FINISH: split-K epilogue for *io splits.
template <typename T, bool DUAL, int EPI>
static void dense_t(const GemmDesc& d, hipStream_t st, DenseOp op, long* io) {
    if (op == OP_FINISH) {
        finish_dense<T, DUAL, EPI>(d, (int)*io, st);
        return;
    }
    with_core<DUAL, EPI, T>(d, [&](auto core) {
        using C = decltype(core);
        if (op == OP_NEED) *io = part_floats<C, T, DUAL, EPI>(d);
        else *io = launch_dense<C, T, DUAL, EPI>(d, st);
    });
}

template <typename T>
static void gemm_t(const GemmDesc& d, hipStream_t st, DenseOp op, long* io) {
    switch (d.epi) {
        case GEMM_STORE_F32: dense_t<T, false, EPI_F32>(d, st, op, io); break;
        case GEMM_STORE_BF16: dense_t<T, false, EPI_BF16>(d, st, op, io); break;
        case GEMM_ADD_F32: dense_t<T, false, EPI_ADD_F32>(d, st, op, io); break;
        case GEMM_SWIGLU:
            if (d.out_f32) dense_t<T, true, EPI_SWIGLU_F32>(d, st, op, io);
            else dense_t<T, true, EPI_SWIGLU_BF16>(d, st, op, io);
            break;
        case GEMM_LMHEAD: dense_t<T, false, EPI_LMHEAD>(d, st, op, io); break;
    }
}

static void gemm_op(const GemmDesc& d, hipStream_t st, DenseOp op, long* io) {
    switch (d.dtype) {
        case DT_F32: gemm_t<float>(d, st, op, io); break;
        case DT_BF16: gemm_t<bf16_t>(d, st, op, io); break;
        case DT_FP8: gemm_t<fp8_t>(d, st, op, io); break;
    }
}

template <typename T, template <typename, bool> class G>
static void grouped_with(const GemmDesc& d, hipStream_t st) {
    switch (d.epi) {
        case GEMM_SWIGLU:
            if (d.out_f32) launch_grouped<G<T, true>, T, EPI_SWIGLU_F32>(d, st);
            else launch_grouped<G<T, true>, T, EPI_SWIGLU_BF16>(d, st);
            break;
        case GEMM_STORE_F32: launch_grouped<G<T, false>, T, EPI_F32>(d, st); break;
        case GEMM_STORE_BF16: launch_grouped<G<T, false>, T, EPI_BF16>(d, st); break;
        default: break;
    }
}

// The tile family must match the m-tile height the routing used
// (grouped_bm with the same assignment count).
template <typename T>
static void grouped_t(const GemmDesc& d, hipStream_t st) {
    if constexpr (std::is_same_v<T, bf16_t>) {
        if (grouped_huge(d.dtype, d.M, d.E)) {
            grouped_with<T, CoreGX>(d, st);
            return;
        }
    }
    if (grouped_large(d.M, d.E)) grouped_with<T, CoreGL>(d, st);
    else grouped_with<T, CoreG>(d, st);
}

int gemm_main(const GemmDesc& d, hipStream_t st) {
    long splits = 1;
    gemm_op(d, st, OP_LAUNCH, &splits);
    return (int)splits;
}

void gemm_splitk_finish(const GemmDesc& d, int splits, hipStream_t st) {
    long s = splits;
    if (splits > 1) gemm_op(d, st, OP_FINISH, &s);
}

long gemm_splitk_floats(const GemmDesc& d) {
    long need = 0;
    gemm_op(d, nullptr, OP_NEED, &need);
    return need;
}

void gemm_grouped(const GemmDesc& d, hipStream_t st) {
    switch (d.dtype) {
        case DT_F32: grouped_t<float>(d, st); break;
        case DT_BF16: grouped_t<bf16_t>(d, st); break;
        case DT_FP8: grouped_t<fp8_t>(d, st); break;
    }
}

int gemm_variants() { return GEMM_VARIANTS; }

// ------------------------------------------------------- weight packing --

long packed_rows(int N) { return (long)(N + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS; }

long packed_weight_bytes(int eb, int batch, int N, int K) { return (long)batch * packed_rows(N) * K * eb; }

// One thread per 16-byte chunk of the packed output: chunk c of matrix b lies
// in block (g, kt) at row r of the block; rows past N are zero.
__global__ __launch_bounds__(256) void pack_weight_kernel(const uint8_t* src, uint8_t* dst, int N, long row_bytes,
                                                          int nkt, long chunks_per_matrix, long total) {
    const long c = (long)blockIdx.x * 256 + threadIdx.x;
    if (c >= total) return;
    const long b = c / chunks_per_matrix, i = c % chunks_per_matrix;
    const long blk = i / (TILE_BYTES / 16);
    const int in = (int)(i % (TILE_BYTES / 16));
    const int r = in / (BKB / 16), ch = in % (BKB / 16);
    const long g = blk / nkt, kt = blk % nkt;
    const long n = g * TILE_ROWS + r;
    uint4 v = {0u, 0u, 0u, 0u};
    if (n < N) v = *(const uint4*)(src + (b * N + n) * row_bytes + kt * BKB + ch * 16);
    *(uint4*)(dst + c * 16) = v;
}

void pack_weight(int eb, int batch, int N, int K, const void* src, void* dst, hipStream_t st) {
    const long row_bytes = (long)K * eb;
    const int nkt = (int)(row_bytes / BKB);
    const long per = packed_rows(N) * row_bytes / 16;
    const long total = per * batch;
    if (total == 0) return;
    launch(pack_weight_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, (const uint8_t*)src,
           (uint8_t*)dst, N, row_bytes, nkt, per, total);
}

int lm_head_tile_n(int M) {
    return M <= 64 ? CoreHs<bf16_t>::BN / CoreHs<bf16_t>::WN : CoreHw<bf16_t>::BN / CoreHw<bf16_t>::WN;
}

}  // namespace dlm
