// MX expert weights (OCP Microscaling Formats v1.0: elements in blocks of 32
// sharing one E8M0 power-of-two scale), in two element formats: MXFP4 (E2M1,
// 4 bits) and MXFP6 (E2M3, 6 bits).  The packed layout, its packer, and the
// grouped expert GEMM that reads it.
//
// Arithmetic: weights-only quantisation.  Each weight is its element value
// times its block's scale, widened exactly to bf16 in registers
// (v_cvt_scalef32_pk_bf16_fp4 / v_cvt_scalef32_pk32_bf16_fp6: an E2M1 or E2M3
// value times a power of two is a bf16 value unless it leaves bf16's range),
// multiplied with the bf16 activations on the bf16 MFMA, fp32 accumulation --
// the same products and sums as a bf16 model whose expert weights are the
// decoded MX values.  Only the bytes in HBM shrink: 4.25 or 6.25 bits a weight.
//
// Packed layout of one [N, K] matrix (K a multiple of 128, N padded to a
// multiple of 16 with zero codes), nT = K / 128 super-steps of 128 elements,
// RB = 128 * bits / 8 code bytes per row and super-step (64 or 96):
//   codes:  block (g, t) of 16 rows x RB bytes at byte (g * nT + t) * 16 RB;
//           row r of the block at +RB r holds elements [128 t, 128 t + 128)
//           of row 16 g + r as in the row-major codes (MXFP4: two per byte,
//           the even element in the low nibble; MXFP6: four per 3 bytes,
//           element 4i + j at bits 6j of the little-endian 24-bit group i),
//           moved whole.
//   scales: block (g, t) of 64 bytes at byte (g * nT + t) * 64; byte r + 16 j
//           is the E8M0 code of row 16 g + r, elements [128 t + 32 j, + 32).
// Experts follow one another.  A wave reads one code block per super-step and
// 16-row tile, lane l taking row l % 16, elements 32 (l / 16) .. + 32 -- one
// scale block: 16 bytes (MXFP4, one load) or 24 (MXFP6, three 8-byte loads)
// -- and the 64 scale bytes with one byte per lane, all contiguous.
//
// The MFMA's K order inside a super-step is permuted, identically for both
// operands: MFMA k-step s (of 4) takes, on lane group q = l / 16, elements
// 32 q + 8 s .. + 8 of the lane's own codes, so each lane widens the codes it
// loaded without any exchange; the activation rows are read from LDS at the
// same element offsets.
//
// Data movement.  A workgroup is NW compute waves plus NPROD producer waves.
// The producers copy the expert m-tile's activation rows (gathered through the
// routing permutation; only the rows the tile holds) into an LDS ring of
// NBUF chunks of SPC super-steps of K, NBUF - 1 chunks ahead of the compute
// waves, with global_load_lds; one barrier per chunk.  The compute waves
// stream their weight tiles from HBM straight into registers, D = P * SPC
// super-steps ahead, so their vmcnt counts only their own weight loads.  Wave
// w owns TNW 16-column tiles (of both weights for the SwiGLU pair); all waves
// share the A chunk in LDS.
#include "common.h"
#include "kernels.h"

namespace dlm {

constexpr int MX_SUPER = 128;        // K elements per super-step
constexpr int MX_SCALE_BLOCK = 64;   // scale bytes per (16 rows, super-step)
constexpr int MX_BM = 64;            // expert m-tile rows

int mx_grouped_bm() { return MX_BM; }

long mx_code_bytes(int bits, int N, int K) { return packed_rows(N) * (long)K * bits / 8; }
long mx_scale_bytes(int N, int K) { return packed_rows(N) * (long)K / 32; }

// ------------------------------------------------------------- packing --

// One thread per 8 bytes of packed codes: block (b, g, t) of 16 rows x rb
// bytes, 8-byte piece p of the block = row p / (rb / 8), bytes 8 (p % (rb /
// 8)) .. + 8 of the row's rb.
__global__ __launch_bounds__(256) void mx_pack_codes_kernel(const uint8_t* src, uint8_t* dst, int N, int K, int rb,
                                                            long per_matrix, long total) {
    const long c = (long)blockIdx.x * 256 + threadIdx.x;
    if (c >= total) return;
    const int nT = K / MX_SUPER, ppr = rb / 8;
    const long b = c / per_matrix, i = c % per_matrix;
    const long blk = i / (16 * ppr);
    const int p = (int)(i % (16 * ppr));
    const long g = blk / nT, t = blk % nT;
    const long n = g * 16 + p / ppr;
    uint2 v = {0u, 0u};
    if (n < N) v = *(const uint2*)(src + (b * N + n) * (long)nT * rb + t * rb + (p % ppr) * 8);
    *(uint2*)(dst + c * 8) = v;
}

// One thread per packed scale byte: block (b, g, t), byte r + 16 j.  Rows past
// N (zero codes) get code 127 (scale 1).
__global__ __launch_bounds__(256) void mx_pack_scales_kernel(const uint8_t* src, uint8_t* dst, int N, int K,
                                                             long per_matrix, long total) {
    const long c = (long)blockIdx.x * 256 + threadIdx.x;
    if (c >= total) return;
    const int nT = K / MX_SUPER;
    const long b = c / per_matrix, i = c % per_matrix;
    const long blk = i / 64;
    const int p = (int)(i % 64);
    const long g = blk / nT, t = blk % nT;
    const long n = g * 16 + p % 16;
    dst[c] = n < N ? src[(b * N + n) * (long)(K / 32) + t * 4 + p / 16] : (uint8_t)127;
}

void mx_pack(int bits, int batch, int N, int K, const void* codes, const void* scales, void* dst_codes,
             void* dst_scales, hipStream_t st) {
    const long pc = mx_code_bytes(bits, N, K) / 8, ps = mx_scale_bytes(N, K);
    if (pc * batch > 0)
        launch(mx_pack_codes_kernel, dim3((unsigned)((pc * batch + 255) / 256)), dim3(256), 0, st,
               (const uint8_t*)codes, (uint8_t*)dst_codes, N, K, MX_SUPER * bits / 8, pc, pc * batch);
    if (ps * batch > 0)
        launch(mx_pack_scales_kernel, dim3((unsigned)((ps * batch + 255) / 256)), dim3(256), 0, st,
               (const uint8_t*)scales, (uint8_t*)dst_scales, N, K, ps, ps * batch);
}

// ------------------------------------------------------- grouped GEMM --

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x32_t __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// E8M0 code -> its scale 2^(e - 127) as fp32 (code 0 is 2^-127, an fp32
// subnormal; 255 is NaN).  Branch-free: ldexp, then one select.
__device__ __forceinline__ float e8m0_scale(uint32_t e) {
    const float s = __builtin_amdgcn_ldexpf(1.0f, (int)e - 127);
    return e == 255u ? __uint_as_float(0x7fc00000u) : s;
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times
// `scale`, as eight bf16 in element order.
__device__ __forceinline__ bf16x8 widen_fp4x8(uint32_t w, float scale) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
    const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
    return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// A lane's codes of one super-step and tile (32 elements, one scale block).
template <int BITS> struct MxCodes;
template <> struct MxCodes<4> {
    static constexpr int LOADS = 1;                          // global loads per super-step
    u32x4 w;
    __device__ __forceinline__ void load(const uint8_t* p) { w = *(const u32x4*)p; }
};
template <> struct MxCodes<6> {
    static constexpr int LOADS = 3;
    uint2 w[3];
    __device__ __forceinline__ void load(const uint8_t* p) {
#pragma unroll
        for (int i = 0; i < 3; ++i) w[i] = *(const uint2*)(p + 8 * i);
    }
};

struct MxArgs {
    const uint8_t* A; long lda;          // bf16 rows, lda in bytes
    const int* gather; int gather_div;   // A row of permuted row p = gather[p] / gather_div (nullable)
    const uint8_t* B; const uint8_t* B2; // packed codes (B2: the SwiGLU pair's second weight)
    const uint8_t* S; const uint8_t* S2; // packed scales
    long b_stride, s_stride;             // bytes between experts
    const int* offs; const int* tile_start;
    int E, N, K;
    void* C; long ldc;                   // elements
};

template <int BITS, bool DUAL, int NW, int TNW, int SPC, int P, int NBUF, int NPROD>
struct MxCfg {
    static constexpr int FMT = BITS;                     // element bits: 4 (E2M1) or 6 (E2M3)
    static constexpr int RB = MX_SUPER * BITS / 8;       // code bytes per row and super-step
    static constexpr int CODE_BLOCK = 16 * RB;           // code bytes per (16 rows, super-step)
    static constexpr int LPG = (MxCodes<BITS>::LOADS + 1) * TNW * (DUAL ? 2 : 1);   // loads per super-step
    static constexpr bool TWO = DUAL;
    static constexpr int NWAVES = NW, TN = TNW, CH = SPC, D = P * SPC, NA = NBUF, NP = NPROD;
    static constexpr int NB = TNW * (DUAL ? 2 : 1);      // weight tiles per wave
    static constexpr int BN = NW * TNW * 16;             // columns per workgroup
    static constexpr int RS = SPC * MX_SUPER * 2;        // LDS bytes per A row and chunk
    static constexpr int ABUF = MX_BM * RS;              // one LDS buffer
    static constexpr int THREADS = (NW + NPROD) * WAVE;
    static_assert(RS <= 1024 && 1024 % RS == 0, "a 1 KB DMA covers whole rows");
    static_assert(LPG * (D - 1) < 64, "vmcnt");
    static_assert(NBUF >= 2 && NBUF * ABUF <= 160 * 1024, "A ring fits LDS");
};

// s_waitcnt vmcnt <= n for a runtime n (the counter never exceeds 63, so
// n >= 63 needs no wait).
template <int N>
__device__ __forceinline__ void wait_vm_le(int n) {
    if constexpr (N == 0) {
        wait_vm<0>();
    } else {
        if (n >= N) wait_vm<N>();
        else wait_vm_le<N - 1>(n);
    }
}

// The producer: chunk c (super-steps [c SPC, c SPC + SPC) clipped to nT) of
// the tile's rows into buffer c % NBUF (the ring keeps NBUF - 1 chunks in
// flight ahead of the compute waves).  1 KB per instruction = 1024 / RS rows;
// lane l fills LDS bytes 16 l .. of the instruction's kilobyte, i.e. row
// R = I * (1024 / RS) + 16 l / RS and physical chunk q' = (16 l % RS) / 16, from
// the row's logical chunk q' ^ (R & 15) (the XOR swizzle the compute waves'
// reads undo).  Rows past the tile's are not loaded (no instruction covers only
// such rows; the rest read the tile's last row); 16-byte chunks past K read the
// row's last chunk -- neither is used.
template <class G>
__device__ __forceinline__ void mx_produce(uint8_t* smem, const MxArgs& a, int c, int rows, int nT,
                                           int my_src, int lane, int pw) {
    constexpr int RPI = 1024 / G::RS;                 // rows per instruction
    const int ninst = (rows + RPI - 1) / RPI;
    uint8_t* buf = smem + (c % G::NA) * G::ABUF;
    const long kbytes = (long)a.K * 2;
    for (int I = pw; I < ninst; I += G::NP) {
        const int R = I * RPI + (lane * 16) / G::RS;
        const int qp = ((lane * 16) % G::RS) / 16;
        const int q = qp ^ (R & 15);
        const long src_row = __shfl(my_src, min(R, rows - 1), WAVE);   // tile row R's source row
        long off = (long)c * G::RS + q * 16;
        off = off < kbytes ? off : kbytes - 16;
        __builtin_amdgcn_global_load_lds((const void*)(a.A + src_row * a.lda + off), (lds_ptr)(buf + I * 1024), 16,
                                         0, 0);
    }
    (void)nT;
}

template <class G, int TMA>
__device__ __forceinline__ void mx_compute(const uint8_t* smem, const MxArgs& a, int ex, int m0, int mlim, int n0,
                                           int nT, int wave, int lane) {
    constexpr int NB = G::NB, D = G::D, SPC = G::CH;
    // this wave's weight tiles: b < TN -> first weight, column tile j = b;
    // b >= TN -> second weight, j = b - TN
    const uint8_t* cb[NB];
    const uint8_t* sb[NB];
    const int colw = n0 + wave * G::TN * 16;
    const int gmax = (a.N - 1) / 16;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int j = b % G::TN;
        const int g = min((colw + j * 16) / 16, gmax);      // tiles past N read the last (not stored)
        const bool second = G::TWO && b >= G::TN;
        cb[b] = (second ? a.B2 : a.B) + (long)ex * a.b_stride + ((long)g * nT) * G::CODE_BLOCK + (lane % 16) * G::RB +
                (lane / 16) * (G::RB / 4);
        sb[b] = (second ? a.S2 : a.S) + (long)ex * a.s_stride + ((long)g * nT) * MX_SCALE_BLOCK + lane;
    }
    f32x4 acc[TMA][NB];
#pragma unroll
    for (int i = 0; i < TMA; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    MxCodes<G::FMT> code[D][NB];
    uint32_t sc[D][NB];
    auto issue = [&](int t, MxCodes<G::FMT> (&cd)[NB], uint32_t (&s)[NB]) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            cd[b].load(cb[b] + (long)t * G::CODE_BLOCK);
            s[b] = sb[b][(long)t * MX_SCALE_BLOCK];
        }
    };
    const int r = lane % 16, q4 = 4 * (lane / 16);
    // super-step t from register group p: A chunk t / SPC from LDS
    auto step = [&](int t, int p) {
        const uint8_t* abuf = smem + ((t / SPC) % G::NA) * G::ABUF;
        const int u = t % SPC;
        float scale[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) scale[b] = e8m0_scale(sc[p][b]);
        // MXFP6: the lane's 32 codes of each tile widened at once (elements 8 s
        // .. + 8 feed k-step s)
        bf16x32_t w6[G::FMT == 6 ? NB : 1];
        if constexpr (G::FMT == 6) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const uint2* c = code[p][b].w;
                w6[b] = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(u32x6{c[0].x, c[0].y, c[1].x, c[1].y, c[2].x, c[2].y},
                                                                      scale[b]);
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 af[TMA];
            const int q = u * 16 + q4 + s;                    // logical 16-byte chunk of the row
#pragma unroll
            for (int i = 0; i < TMA; ++i) af[i] = *(const bf16x8*)(abuf + (i * 16 + r) * G::RS + ((q ^ r) << 4));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                bf16x8 bf;
                if constexpr (G::FMT == 4) {
                    bf = widen_fp4x8(code[p][b].w[s], scale[b]);
                } else {
                    const bf16x32_t& v = w6[b];
                    bf = bf16x8{v[8 * s], v[8 * s + 1], v[8 * s + 2], v[8 * s + 3], v[8 * s + 4], v[8 * s + 5],
                                v[8 * s + 6], v[8 * s + 7]};
                }
#pragma unroll
                for (int i = 0; i < TMA; ++i)
                    acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf, acc[i][b], 0, 0, 0);
            }
        }
    };
    // Every step issues one group (the super-step D ahead, or the last one
    // again near the end), so the count of loads in flight is the same on
    // every path: D - 1 groups after the one a step waits for.
#pragma unroll
    for (int p = 0; p < D; ++p) issue(min(p, nT - 1), code[p], sc[p]);
    int t0 = 0;
    for (; t0 + D <= nT; t0 += D) {
#pragma unroll
        for (int p = 0; p < D; ++p) {
            const int t = t0 + p;
            wait_vm<G::LPG * (D - 1)>();
            // no instruction of a later step is scheduled before this wait
            // (the compiler would wait for that step's loads here)
            __builtin_amdgcn_sched_barrier(0);
            if (p % SPC == 0) stage_barrier();                // chunk t / SPC is in LDS
            step(t, p);
            issue(min(t + D, nT - 1), code[p], sc[p]);
        }
    }
    // fewer than D super-steps left: their groups are in flight
    wait_vm<0>();
#pragma unroll
    for (int p = 0; p < D; ++p) {
        const int t = t0 + p;
        if (t < nT) {
            if (p % SPC == 0) stage_barrier();
            step(t, p);
        }
    }

    // epilogue: D[4 (l / 16) + v][l % 16] of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < TMA; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = m0 + i * 16 + (lane / 16) * 4 + v;
            if (row >= mlim) continue;
#pragma unroll
            for (int j = 0; j < G::TN; ++j) {
                const int col = colw + j * 16 + lane % 16;
                if (col >= a.N) continue;
                const long off = (long)row * a.ldc + col;
                if constexpr (G::TWO) {
                    ((bf16_t*)a.C)[off] = f32_to_bf16(silu_f(acc[i][j][v]) * acc[i][G::TN + j][v]);
                } else {
                    ((float*)a.C)[off] = acc[i][j][v];
                }
            }
        }
}

template <class G>
__global__ __launch_bounds__(G::THREADS) void mx_grouped_kernel(MxArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t smem[G::NA * G::ABUF];
    // live tiles dealt to the 8 XCDs in equal contiguous ranges (as the bf16
    // grouped GEMM): m-tiles of one weight tile adjacent, one L2
    const int nt_n = (a.N + G::BN - 1) / G::BN;
    const int mtiles = a.tile_start[a.E];
    const int live = mtiles * nt_n;
    const int per = (live + 7) / 8;
    const int slot = blockIdx.x / 8;
    if (slot >= per) return;
    const int lin = (blockIdx.x % 8) * per + slot;
    if (lin >= live) return;
    const int nt = lin / mtiles, mt = lin % mtiles;
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (a.tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int ex = lo;
    const int m0 = a.offs[ex] + (mt - a.tile_start[ex]) * MX_BM;
    const int mlim = a.offs[ex + 1];
    const int rows = min(MX_BM, mlim - m0);              // >= 1 for a live tile
    const int n0 = nt * G::BN;
    const int nT = a.K / MX_SUPER;
    const int nch = (nT + G::CH - 1) / G::CH;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
    const int lane = threadIdx.x % WAVE;

    if (wave >= G::NWAVES) {
        const int pw = wave - G::NWAVES;                  // producer pw issues loads pw, pw + NP, ...
        // source row of tile row `lane` (rows past the tile: its last row)
        const int pr = m0 + min(lane, rows - 1);
        const int my_src = a.gather ? a.gather[pr] / a.gather_div : pr;
        constexpr int RPI = 1024 / G::RS;
        const int ninst = ((rows + RPI - 1) / RPI - pw + G::NP - 1) / G::NP;   // this producer's loads per chunk
        for (int c = 0; c < G::NA - 1 && c < nch; ++c) mx_produce<G>(smem, a, c, rows, nT, my_src, lane, pw);
        for (int c = 0; c < nch; ++c) {
            // chunk c landed: only the chunks issued after it may be in flight
            wait_vm_le<63>(ninst * (min(nch - 1, c + G::NA - 2) - c));
            stage_barrier();                              // chunk c ready; everyone done with chunk c - 1
            if (c + G::NA - 1 < nch) mx_produce<G>(smem, a, c + G::NA - 1, rows, nT, my_src, lane, pw);
        }
        return;
    }
    switch ((rows + 15) / 16) {
        case 1: mx_compute<G, 1>(smem, a, ex, m0, mlim, n0, nT, wave, lane); break;
        case 2: mx_compute<G, 2>(smem, a, ex, m0, mlim, n0, nT, wave, lane); break;
        case 3: mx_compute<G, 3>(smem, a, ex, m0, mlim, n0, nT, wave, lane); break;
        default: mx_compute<G, 4>(smem, a, ex, m0, mlim, n0, nT, wave, lane); break;
    }
}

// Variants (the test hook may force one): 0 = the model's choice.  Compute
// waves x column tiles per wave, super-steps per A chunk, chunks of weight
// prefetch, chunks in the A ring, producer waves.  Several producer waves
// matter most: one wave issuing every A copy was the bottleneck (a sweep on
// the 26B-class canvas step's expert shapes, 2048 assignments over 58
// experts: 69 -> 45 us for gate/up with four).
template <int BITS, bool DUAL, class F>
static bool mx_with_variant(int v, F f) {
    switch (v) {
        case 0:   // 6-bit codes hold 50% more registers in flight: the pair takes 8 waves x 1 tile
            if constexpr (DUAL && BITS == 4) f(MxCfg<BITS, DUAL, 4, 2, 2, 1, 2, 4>{});
            else if constexpr (DUAL) f(MxCfg<BITS, DUAL, 8, 1, 2, 1, 2, 4>{});
            else f(MxCfg<BITS, DUAL, 8, 2, 2, 1, 2, 4>{});
            return true;
        case 1: f(MxCfg<BITS, DUAL, 4, DUAL ? 2 : 4, 2, 1, 3, 4>{}); return true;
        case 2: f(MxCfg<BITS, DUAL, 4, DUAL ? 2 : 4, 1, 3, 4, 4>{}); return true;
        case 3: f(MxCfg<BITS, DUAL, 8, DUAL ? 1 : 2, 2, 2, 4, 4>{}); return true;
        case 4: f(MxCfg<BITS, DUAL, 4, DUAL ? 2 : 4, 2, 1, 4, 1>{}); return true;
        case 5: f(MxCfg<BITS, DUAL, 4, DUAL ? 2 : 4, 2, 1, 2, 2>{}); return true;
        default: return false;
    }
}
constexpr int MX_VARIANTS = 5;
int mx_variants() { return MX_VARIANTS; }

template <int BITS, bool DUAL>
static void mx_launch(const MxDesc& d, hipStream_t st) {
    mx_with_variant<BITS, DUAL>(d.variant, [&](auto g) {
        using G = decltype(g);
        MxArgs a;
        a.A = (const uint8_t*)d.A; a.lda = d.lda * 2;
        a.gather = d.gather; a.gather_div = d.gather_div;
        a.B = (const uint8_t*)d.B; a.B2 = (const uint8_t*)d.B2;
        a.S = (const uint8_t*)d.S; a.S2 = (const uint8_t*)d.S2;
        a.b_stride = d.b_stride; a.s_stride = d.s_stride;
        a.offs = d.offs; a.tile_start = d.tile_start;
        a.E = d.E; a.N = d.N; a.K = d.K;
        a.C = d.C; a.ldc = d.ldc;
        const long max_mtiles = (d.M + MX_BM - 1) / MX_BM + d.E;
        const long grid = (max_mtiles * ((d.N + G::BN - 1) / G::BN) + 7) / 8 * 8;
        if (d.M == 0 || grid == 0) return;
        launch((mx_grouped_kernel<G>), dim3((unsigned)grid), dim3(G::THREADS), 0, st, a);
    });
}

void mx_grouped(const MxDesc& d, hipStream_t st) {
    if (d.bits == 6) {
        if (d.swiglu) mx_launch<6, true>(d, st);
        else mx_launch<6, false>(d, st);
    } else {
        if (d.swiglu) mx_launch<4, true>(d, st);
        else mx_launch<4, false>(d, st);
    }
}

}  // namespace dlm
