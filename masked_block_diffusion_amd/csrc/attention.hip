// Attention over the KV cache for gfx950.
//
// Denoising ("block") mode: every canvas query sees every cached key [0, T) and
// every canvas key [T, T + C) -- bidirectional inside the canvas, full to the
// prefix.  Prefill ("causal") mode: the query at position p sees keys [0, p].
// Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
//
// Cache: per (layer, KV head) keys as rows and values transposed, contiguous
// or in 64-token pages (kvcache.h); a 64-key tile is one KV block (one page).
//
// bf16 kernel (flash-style, online softmax in fp32):
//   * A workgroup owns one KV head of one request, NW * 32 "query rows" (pairs
//     of canvas position and query head of that KV head's group; 32 per wave,
//     two 16-row MFMA blocks; NW = 8 waves for dh 128) and a range of 64-key
//     tiles, so all the group's queries share every K / V^T tile staged in LDS.
//   * K and V^T tiles are plain row-major copies, so they go global -> LDS by
//     global_load_lds_dwordx4 (no register staging) into an NS-stage ring
//     (NS - 1 tiles in flight while one is computed, one barrier per tile); the
//     16-byte chunks of a row are XOR-swizzled by the row index so the fragment
//     reads of 16 rows spread over the LDS banks.  Per-tile work is a short
//     dependent chain (scores, softmax, P V), so the deep ring and two waves
//     per SIMD are what keep the MFMA pipes fed.
//   * Scores are computed transposed, S^T = K Q^T, with 16x16x32 bf16 MFMAs:
//     one query per lane column, so the online-softmax statistics are per-lane
//     scalars and P^T is already laid out as the B operand of O^T = V^T P^T.
//     The rows of a 16-key score block are taken in a permuted key order
//     (key_of), chosen so the 8 probabilities a lane feeds to one P V MFMA are
//     8 consecutive keys: its V^T operand is then one 16-byte LDS read.
//   * P enters the P V MFMAs as two bf16 terms (hi = bf16(p), lo = bf16(p -
//     hi)), so P V is taken at fp32 level (relative error ~2^-16 per
//     probability) like the softmax itself; a single bf16 term would add a
//     2^-9 rounding of every probability that the model does not have.
//   * Long key ranges are split across workgroups (split-KV) when the
//     (request, KV head, query block) workgroups alone are too few for the
//     chip, in denoising and in prefill; partial (max, sum, unnormalised O)
//     are merged by a second kernel in fixed split order.
//   * Keys past the end of the range are never read from memory the caller
//     has not written: their K rows are fetched from the tile's first key (and
//     masked), and
//     V^T chunks reaching past the end are zeroed in LDS by the lane that
//     fetched them (unwritten cache slots may hold any bit pattern, and 0 * NaN
//     would poison the sum).
// fp32 kernel (fp32 models): one thread per (query, head), online softmax,
// fp32 throughout.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "kvcache.h"

namespace dlm {

constexpr int KT = 64;           // keys per tile
constexpr int MAX_SPLITS = 16;
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
    const bf16_t* q;             // [rows, hq, dh]
    SeqTab seqs;
    int layer, hq, hkv, group;
    int causal;
    int n_qblocks;               // per (request, kv head)
    uint8_t order[MAX_SEQS];     // requests in dispatch order: longest key range first
    int n_splits;
    int tiles_per_split;
    float scale_log2;            // dh^-1/2 * log2(e)
    bf16_t* out;                 // [rows, hq, dh] (n_splits == 1)
    float* o_part;               // [n_splits, rows, hq, dh]
    float* ml_part;              // [n_splits, rows, hq, 2]
    int rows;
};
static_assert(MAX_SEQS <= 256, "request indices fit AttnArgs::order");

template <int DH>
struct AttnShape {
    static constexpr int NW = DH >= 128 ? 8 : 4;     // waves per workgroup
    static constexpr int QBN = 2;                    // 16-row query blocks per wave
    static constexpr int QW = 16 * QBN;              // query rows per wave
    static constexpr int QB = NW * QW;               // query rows per workgroup
    static constexpr int NSTAGE = 4;                 // ring stages
    static constexpr int KROWB = DH * 2;             // bytes per K row
    static constexpr int KCH = DH / 8;               // 16-byte chunks per K row
    static constexpr int KBYTES = KT * KROWB;
    static constexpr int VROWB = KT * 2;             // bytes per V^T row (one tile's keys)
    static constexpr int VCH = KT / 8;
    static constexpr int VBYTES = DH * VROWB;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int ROUND = NW * 1024;          // bytes one load instruction of every wave fills
    static constexpr int KLPT = KBYTES / ROUND;      // K loads per thread per stage
    static constexpr int LPT = STAGE / ROUND;        // all loads per thread per stage
    static constexpr int NS = DH / 32;               // MFMA k-steps over dh
    static constexpr int ND = DH / 16;               // dh sub-tiles of O^T
    static_assert(KBYTES % ROUND == 0 && VBYTES % ROUND == 0, "whole load rounds per operand");
    static_assert((NSTAGE - 2) * LPT < 64, "vmcnt");
};

// Tile-relative key of row i (0..15) of 16-key score block u (0..3): lane group
// g holds rows 4g..4g+3 of every block, i.e. keys 32*(u/2) + 8g + 4*(u%2) + v,
// so blocks 2h and 2h+1 together give it keys 32h + 8g .. 32h + 8g + 7.
__device__ __forceinline__ int key_of(int u, int i) {
    return 32 * (u >> 1) + 8 * (i >> 2) + 4 * (u & 1) + (i & 3);
}

// Maximum of x over lanes i and i ^ 16 (resp. i ^ 32), by the gfx950 row
// swaps: swapping a value with itself leaves each lane its own value in one
// half of the returned pair and its partner's in the other.
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// 2^x by the hardware instruction (results below 2^-126 flush to 0, which
// only drops terms far below the row's largest probability)
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int DH>
__global__ __launch_bounds__(AttnShape<DH>::NW * WAVE) void attn_bf16_kernel(AttnArgs a) {
    using S = AttnShape<DH>;
    constexpr int QB = S::QB, QW = S::QW, QBN = S::QBN;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[S::NSTAGE * S::STAGE];

    int b = blockIdx.x;
    const int split = b % a.n_splits; b /= a.n_splits;
    const int qblk = b % a.n_qblocks; b /= a.n_qblocks;
    const int kvh = b % a.hkv; b /= a.hkv;
    const int sq = a.order[b];
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int g = lane / 16, li = lane % 16;
    const int per = a.seqs.per_seq;
    const int T = a.seqs.T[sq];
    const int n_keys = T + per;

    // this lane's two query rows (one per 16-row block): (canvas row qi, query
    // head) of query row qr; recomputed where needed rather than kept live
    const int nq = per * a.group;
    auto qrow = [&](int qb) { return qblk * QB + wave * QW + qb * 16 + li; };
    bf16x8 qf[QBN][S::NS];
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
        const int qr = qrow(qb);
        const bool ok = qr < nq;
        const long orow = (long)sq * per + (ok ? qr / a.group : 0);
        const int qh = kvh * a.group + (ok ? qr % a.group : 0);
#pragma unroll
        for (int s = 0; s < S::NS; ++s)
            qf[qb][s] = ok ? *(const bf16x8*)(a.q + (orow * a.hq + qh) * DH + 32 * s + 8 * g) : bf16x8{};
    }

    // key range of this workgroup
    int kend = n_keys;
    if (a.causal) {
        const int last = min(nq - 1, qblk * QB + QB - 1);
        kend = min(n_keys, T + last / a.group + 1);
    }
    const int ntiles = (kend + KT - 1) / KT;
    const int t0 = split * a.tiles_per_split;
    const int t1 = min(ntiles, t0 + a.tiles_per_split);
    // first query position of this wave: tiles reaching past it need the causal mask
    const int wave_pos0 = T + min(qblk * QB + wave * QW, nq - 1) / a.group;

    // DMA assignment: load j of this thread fills stage bytes [I*1024 + lane*16, +16),
    // I = j*NW + wave; K rows first (row, swizzled chunk), then V^T rows (dh, chunk).
    auto lrow = [&](int j) {
        const int off = (j * S::NW + wave) * 1024 + lane * 16;
        return j < S::KLPT ? off / S::KROWB : (off - S::KBYTES) / S::VROWB;
    };
    auto lchunk = [&](int j) {
        const int off = (j * S::NW + wave) * 1024 + lane * 16;
        return j < S::KLPT ? ((off % S::KROWB) / 16) ^ (lrow(j) % S::KCH)
                           : (((off - S::KBYTES) % S::VROWB) / 16) ^ (lrow(j) % S::VCH);
    };
    // tile t is KV block t of the cache (one page when paged); keys at or past
    // kend are fetched from the tile's first key / first chunk instead
    auto issue = [&](int tile, int slot) {
        const int k0 = tile * KT;
        const KVBlock<const bf16_t> kb = kv_block<const bf16_t>(a.seqs, sq, a.layer, a.hkv, kvh, DH, tile);
        uint8_t* st = smem + slot * S::STAGE;
#pragma unroll
        for (int j = 0; j < S::LPT; ++j) {
            const bf16_t* src;
            if (j < S::KLPT) {
                const int key = k0 + lrow(j);
                src = kb.k + (long)(key < kend ? lrow(j) : 0) * DH + lchunk(j) * 8;
            } else {
                const int kc = k0 + 8 * lchunk(j);
                src = kb.vt + (long)lrow(j) * kb.vstride + (kc < kend ? 8 * lchunk(j) : 0);
            }
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(st + (j * S::NW + wave) * 1024), 16, 0, 0);
        }
    };
    // V^T slots of keys >= kend in the tile: zero (after this lane's own loads landed)
    auto zero_tail = [&](int tile, int slot) {
        const int k0 = tile * KT;
        if (k0 + KT <= kend) return;
        uint8_t* st = smem + slot * S::STAGE;
#pragma unroll
        for (int j = S::KLPT; j < S::LPT; ++j) {
            const int nv = kend - (k0 + 8 * lchunk(j));
            if (nv < 8) {
                bf16_t* dst = (bf16_t*)(st + (j * S::NW + wave) * 1024 + lane * 16);
                for (int e = max(nv, 0); e < 8; ++e) dst[e] = 0;
            }
        }
    };

    float m_run[QBN], l_run[QBN];
    f32x4 o[QBN][S::ND];
#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int d = 0; d < S::ND; ++d) o[qb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int lv = li, gv = g;
    // S^T = K Q^T of one tile: 4 blocks of 16 keys, for both query blocks
    auto scores = [&](const uint8_t* ks, f32x4 (&sc)[QBN][4]) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int qb = 0; qb < QBN; ++qb) sc[qb][u] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int R = key_of(u, lv);
#pragma unroll
            for (int s = 0; s < S::NS; ++s) {
                const int c = 4 * s + gv;
                const bf16x8 kf = *(const bf16x8*)(ks + R * S::KROWB + ((c ^ (R % S::KCH)) << 4));
#pragma unroll
                for (int qb = 0; qb < QBN; ++qb) sc[qb][u] = mfma_bf16(kf, qf[qb][s], sc[qb][u]);
            }
        }
    };
    // mask (only tiles that reach past kend or a causal diagonal), then the
    // online softmax per query (= per lane column) of tile t; P in bf16
    auto softmax = [&](const f32x4 (&sc)[QBN][4], int t, bf16x8 (&ph)[QBN][2], bf16x8 (&pl)[QBN][2]) {
        const int k0 = t * KT;
        const bool full = k0 + KT <= kend && !(a.causal && k0 + KT - 1 > wave_pos0);
        // Masked scores x: a select on read (no writes into the MFMA results).
        // Row i = 4 gv + v of score block u is tile key key_of(u, i) =
        // 8 gv + (32 (u / 2) + 4 (u % 2) + v), valid while it is at most the
        // query's last visible key (kend - 1, and its own position if causal).
        float x[QBN][4][4];
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) {
            int kmax = kend - 1;
            if (a.causal) kmax = min(kmax, T + min(qrow(qb), nq - 1) / a.group);
            const int lim = full ? KT : kmax - k0 - 8 * gv;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    x[qb][u][v] = (32 * (u >> 1) + 4 * (u & 1) + v <= lim) ? sc[qb][u][v] : -INFINITY;
        }
        float mt[QBN];
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) {
            const float m01 = fmaxf(fmaxf(x[qb][0][0], x[qb][0][1]), fmaxf(x[qb][0][2], x[qb][0][3]));
            const float m11 = fmaxf(fmaxf(x[qb][1][0], x[qb][1][1]), fmaxf(x[qb][1][2], x[qb][1][3]));
            const float m21 = fmaxf(fmaxf(x[qb][2][0], x[qb][2][1]), fmaxf(x[qb][2][2], x[qb][2][3]));
            const float m31 = fmaxf(fmaxf(x[qb][3][0], x[qb][3][1]), fmaxf(x[qb][3][2], x[qb][3][3]));
            mt[qb] = fmaxf(fmaxf(m01, m11), fmaxf(m21, m31));
        }
        // the four lane groups holding a query's keys: lanes li, li+16, li+32, li+48
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) mt[qb] = max_xor16(mt[qb]);
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) mt[qb] = max_xor32(mt[qb]);
#pragma unroll
        for (int qb = 0; qb < QBN; ++qb) {
            const float m_new = fmaxf(m_run[qb], mt[qb] * a.scale_log2);
            // a query with every key so far masked keeps o = l = 0: use 0 as
            // its reference so exp2(-inf - 0) = 0 and no NaN appears
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = exp2_raw(m_run[qb] - m_use);
            m_run[qb] = m_new;
            // P in key pairs of blocks (2 h2, 2 h2 + 1), straight to bf16
            float ps = 0.f;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                float q0[4], q1[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    q0[v] = exp2_raw(fmaf(x[qb][2 * h2][v], a.scale_log2, -m_use));
                    q1[v] = exp2_raw(fmaf(x[qb][2 * h2 + 1][v], a.scale_log2, -m_use));
                    ph[qb][h2][v] = (__bf16)q0[v];
                    ph[qb][h2][4 + v] = (__bf16)q1[v];
                    pl[qb][h2][v] = (__bf16)(q0[v] - (float)ph[qb][h2][v]);
                    pl[qb][h2][4 + v] = (__bf16)(q1[v] - (float)ph[qb][h2][4 + v]);
                }
                ps += ((q0[0] + q0[1]) + (q0[2] + q0[3])) + ((q1[0] + q1[1]) + (q1[2] + q1[3]));
            }
            l_run[qb] = l_run[qb] * alpha + ps;
            // rescale O only when some query's maximum moved (uniform branch)
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int d = 0; d < S::ND; ++d) o[qb][d] *= alpha;
            }
        }
    };
    // O^T += V^T P^T of one tile: per dh sub-tile, two 32-key MFMA steps
    auto pv = [&](const uint8_t* vs, const bf16x8 (&ph)[QBN][2], const bf16x8 (&pl)[QBN][2]) {
#pragma unroll
        for (int d = 0; d < S::ND; ++d) {
            const int row = d * 16 + lv;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int c = 4 * h2 + gv;
                const bf16x8 vf = *(const bf16x8*)(vs + row * S::VROWB + ((c ^ (row % S::VCH)) << 4));
#pragma unroll
                for (int qb = 0; qb < QBN; ++qb) {
                    o[qb][d] = mfma_bf16(vf, ph[qb][h2], o[qb][d]);
                    o[qb][d] = mfma_bf16(vf, pl[qb][h2], o[qb][d]);
                }
            }
        }
    };

    // One barrier per tile: after it, tile t is visible to every wave and every
    // wave is done with tile t - 1, whose slot takes tile t - 1 + NST.  Tile t
    // sits in slot (t - t0) % NST; NST - 1 tiles are in flight while one is
    // computed.
    constexpr int NST = S::NSTAGE;
#pragma unroll
    for (int i = 0; i < NST - 1; ++i)
        if (t0 + i < t1) issue(t0 + i, i);
    for (int t = t0; t < t1; ++t) {
        const int slot = (t - t0) % NST;
        wait_stages<S::LPT, NST - 2>(min(NST - 2, t1 - 1 - t));   // tile t landed
        zero_tail(t, slot);
        stage_barrier();
        if (t + NST - 1 < t1) issue(t + NST - 1, (t - t0 + NST - 1) % NST);
        const uint8_t* ks = smem + slot * S::STAGE;
        f32x4 sc[QBN][4];
        bf16x8 ph[QBN][2], pl[QBN][2];
        scores(ks, sc);
        softmax(sc, t, ph, pl);
        pv(ks + S::KBYTES, ph, pl);
    }

#pragma unroll
    for (int qb = 0; qb < QBN; ++qb) {
        // row sum across the 4 lane groups holding this query
        float l = l_run[qb];
        l += __shfl_xor(l, 16, WAVE);
        l += __shfl_xor(l, 32, WAVE);
        const int qr = qrow(qb);
        if (qr >= nq) continue;
        const long orow = (long)sq * per + qr / a.group;
        const int qh = kvh * a.group + qr % a.group;
        const long obase = (orow * a.hq + qh) * DH;
        if (a.n_splits == 1) {
            const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int d = 0; d < S::ND; ++d) {
                uint64_t packed = 0;
#pragma unroll
                for (int v = 0; v < 4; ++v) packed |= (uint64_t)f32_to_bf16(o[qb][d][v] * inv) << (16 * v);
                *(uint64_t*)(a.out + obase + d * 16 + 4 * g) = packed;
            }
        } else {
            float* op = a.o_part + (long)split * a.rows * a.hq * DH + obase;
#pragma unroll
            for (int d = 0; d < S::ND; ++d) *(f32x4*)(op + d * 16 + 4 * g) = o[qb][d];
            if (g == 0) {
                float* ml = a.ml_part + ((long)split * a.rows * a.hq + orow * a.hq + qh) * 2;
                ml[0] = m_run[qb];
                ml[1] = l;
            }
        }
    }
}

// Merge split partials: O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j, in
// split order.  One thread per 4 consecutive dh elements of a (row, head); every
// split's loads are issued before the arithmetic.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* o_part, const float* ml_part, int n_splits,
                                                          long pairs, int dh, bf16_t* out) {
    const int tpp = dh / 4;                       // threads per (row, head)
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    const long rh = t / tpp;
    if (rh >= pairs) return;
    const int c = (int)(t % tpp) * 4;
    float m[MAX_SPLITS], l[MAX_SPLITS];
    f32x4 ov[MAX_SPLITS];
#pragma unroll
    for (int j = 0; j < MAX_SPLITS; ++j) {
        if (j < n_splits) {
            const float2 v = *(const float2*)(ml_part + (j * pairs + rh) * 2);
            m[j] = v.x;
            l[j] = v.y;
            ov[j] = *(const f32x4*)(o_part + (j * pairs + rh) * dh + c);
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAX_SPLITS; ++j)
        if (j < n_splits) M = fmaxf(M, m[j]);
    float L = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < MAX_SPLITS; ++j) {
        if (j < n_splits && m[j] != -INFINITY) {
            const float w = exp2f(m[j] - M);
            L += w * l[j];
            acc += w * ov[j];
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint64_t packed = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) packed |= (uint64_t)f32_to_bf16(acc[v] * inv) << (16 * v);
    *(uint64_t*)(out + rh * dh + c) = packed;
}

// fp32 models: one thread per (query row, head).
template <int DH>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* q, SeqTab seqs, int layer, int hq, int hkv,
                                                       int causal, float scale, float* out) {
    const int per = seqs.per_seq;
    const int idx = blockIdx.x * 64 + threadIdx.x;
    const int total = seqs.n * per * hq;
    if (idx >= total) return;
    const int h = idx % hq;
    const int r = idx / hq;
    const int sq = r / per, i = r % per;
    const int T = seqs.T[sq];
    const int pos = T + i;
    const int kvh = h / (hq / hkv);
    const int kend = causal ? pos + 1 : T + per;
    float qv[DH], o[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) {
        qv[c] = q[((long)r * hq + h) * DH + c];
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    KVBlock<const float> b{};
    for (int k = 0; k < kend; ++k) {
        if (k % KV_PAGE == 0) b = kv_block<const float>(seqs, sq, layer, hkv, kvh, DH, k / KV_PAGE);
        const int i = k % KV_PAGE;
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < DH; ++c) s += qv[c] * b.k[(long)i * DH + c];
        s *= scale;
        const float mn = fmaxf(m, s);
        const float al = expf(m - mn);
        const float p = expf(s - mn);
        l = l * al + p;
#pragma unroll
        for (int c = 0; c < DH; ++c) o[c] = o[c] * al + p * b.vt[(long)c * b.vstride + i];
        m = mn;
    }
#pragma unroll
    for (int c = 0; c < DH; ++c) out[((long)r * hq + h) * DH + c] = o[c] / l;
}

// Split-KV only while splits * rows stays within SPLIT_ROWS (bounds the
// partial buffers); each split keeps at least MIN_SPLIT_TILES key tiles; aim
// for about one round of workgroups over the 256 CUs (as many per CU as the
// ring's LDS allows, at most two).
constexpr int SPLIT_ROWS = 4096;
constexpr int MIN_SPLIT_TILES = 2;

static int choose_splits(int target, int base_blocks, int ntiles, int rows) {
    int s = (target + base_blocks - 1) / base_blocks;
    s = min(s, max(1, ntiles / MIN_SPLIT_TILES));
    s = min(s, max(1, SPLIT_ROWS / rows));
    return max(1, min(s, MAX_SPLITS));
}

template <int DH>
static void launch_attn_bf16(AttnArgs& a, int n_seqs, int max_keys, bool causal, int rows,
                             hipStream_t st) {
    using S = AttnShape<DH>;
    constexpr int per_cu = (160 * 1024) / (S::NSTAGE * S::STAGE) >= 2 ? 2 : 1;
    a.n_qblocks = (a.seqs.per_seq * a.group + S::QB - 1) / S::QB;
    // Requests' workgroups are dispatched longest key range first (ties by
    // index), so the short ones fill the tail: 32 requests with prompts of
    // 512 to 4096 tokens, attention 16.2 -> 15.2 ms per step.  Each
    // workgroup's work is unchanged, so are the results.
    for (int i = 0; i < n_seqs; ++i) a.order[i] = (uint8_t)i;
    std::stable_sort(a.order, a.order + n_seqs, [&](uint8_t x, uint8_t y) { return a.seqs.T[x] > a.seqs.T[y]; });
    const int ntiles = (max_keys + KT - 1) / KT;
    const int base = n_seqs * a.hkv * a.n_qblocks;
    // causal (prefill) ranges split too: a query block's keys end at its last
    // position, so later splits of early blocks are empty (written as max
    // -inf, skipped by the merge), and the longest block's work is divided
    a.n_splits = choose_splits(256 * per_cu, base, ntiles, rows);
    a.tiles_per_split = (ntiles + a.n_splits - 1) / a.n_splits;
    a.n_splits = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
    if (a.n_splits < 1) a.n_splits = 1;
    launch(attn_bf16_kernel<DH>, dim3(base * a.n_splits), dim3(S::NW * WAVE), 0, st, a);
}

long attention_work_floats(int rows, int hq, int dh) {
    (void)rows;
    return (long)SPLIT_ROWS * hq * (dh + 2);
}

void attention(const void* q, const SeqTab& seqs, int layer, int n_layers, int hq, int hkv, int dh, bool causal,
               bool f32, void* out, const AttnWork& w, hipStream_t st) {
    (void)n_layers;
    const int rows = seqs.n * seqs.per_seq;
    if (rows <= 0) return;
    if (f32) {
        const int total = rows * hq;
        const float scale = 1.0f / sqrtf((float)dh);
        const dim3 grid((total + 63) / 64);
        if (dh == 32) launch(attn_f32_kernel<32>, grid, dim3(64), 0, st, (const float*)q, seqs, layer, hq, hkv, (int)causal, scale, (float*)out);
        else if (dh == 64) launch(attn_f32_kernel<64>, grid, dim3(64), 0, st, (const float*)q, seqs, layer, hq, hkv, (int)causal, scale, (float*)out);
        else launch(attn_f32_kernel<128>, grid, dim3(64), 0, st, (const float*)q, seqs, layer, hq, hkv, (int)causal, scale, (float*)out);
        return;
    }
    AttnArgs a;
    a.q = (const bf16_t*)q;
    a.seqs = seqs;
    a.layer = layer; a.hq = hq; a.hkv = hkv; a.group = hq / hkv;
    a.causal = causal ? 1 : 0;
    int max_keys = 0;
    for (int i = 0; i < seqs.n; ++i) max_keys = max(max_keys, seqs.T[i] + seqs.per_seq);
    a.scale_log2 = LOG2E / sqrtf((float)dh);
    a.out = (bf16_t*)out;
    a.o_part = w.o_part;
    a.ml_part = w.ml_part;
    a.rows = rows;
    if (dh == 128) launch_attn_bf16<128>(a, seqs.n, max_keys, causal, rows, st);
    else if (dh == 64) launch_attn_bf16<64>(a, seqs.n, max_keys, causal, rows, st);
    else launch_attn_bf16<32>(a, seqs.n, max_keys, causal, rows, st);
    if (a.n_splits > 1) {
        // the merge is a kernel of its own for timing purposes
        LaunchTimer* t = launch_timer();
        launch_timer() = w.merge_timer;
        const long pairs = (long)rows * hq;
        const long threads = pairs * (dh / 4);
        launch(attn_merge_kernel, dim3((threads + 255) / 256), dim3(256), 0, st, w.o_part, w.ml_part,
               a.n_splits, pairs, dh, (bf16_t*)out);
        launch_timer() = t;
    }
}

}  // namespace dlm
