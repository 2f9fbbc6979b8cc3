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
//   * A workgroup owns one KV head of one request, 128 "query rows" (pairs of
//     canvas position and query head of that KV head's group; 32 per wave, two
//     16-row MFMA blocks) and a range of 64-key tiles, so all the group's
//     queries share every K / V^T tile staged in LDS.
//   * K and V^T tiles are plain row-major copies, so they go global -> LDS by
//     global_load_lds_dwordx4 (no register staging) into a two-stage ring; the
//     16-byte chunks of a row are XOR-swizzled by the row index so the fragment
//     reads of 16 rows spread over the LDS banks.
//   * Scores are computed transposed, S^T = K Q^T, with 16x16x32 bf16 MFMAs:
//     one query per lane column, so the online-softmax statistics are per-lane
//     scalars and P^T is already laid out as the B operand of O^T = V^T P^T.
//     The rows of a 16-key score block are taken in a permuted key order
//     (key_of), chosen so the 8 probabilities a lane feeds to one P V MFMA are
//     8 consecutive keys: its V^T operand is then one 16-byte LDS read.
//   * P is fed as two bf16 terms (hi + lo), so P V carries fp32-level precision.
//   * Long key ranges are split across workgroups (split-KV); partial (max,
//     sum, unnormalised O) are merged by a second kernel in fixed split order.
//   * Keys past the end of the range are never read from memory the caller
//     has not written: their K rows are fetched from the tile's first key (and
//     masked), and
//     V^T chunks reaching past the end are zeroed in LDS by the lane that
//     fetched them (unwritten cache slots may hold any bit pattern, and 0 * NaN
//     would poison the sum).
// fp32 kernel (fp32 models): one thread per (query, head), online softmax,
// fp32 throughout.
#include "common.h"
#include "kernels.h"
#include "kvcache.h"

namespace dlm {

constexpr int KT = 64;           // keys per tile
constexpr int QW = 32;           // query rows per wave
constexpr int QB = 4 * QW;       // query rows per workgroup
constexpr int MAX_SPLITS = 16;
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
    const bf16_t* q;             // [rows, hq, dh]
    SeqTab seqs;
    int layer, hq, hkv, group;
    int causal;
    int n_qblocks;               // per (request, kv head)
    int n_splits;
    int tiles_per_split;
    float scale_log2;            // dh^-1/2 * log2(e)
    bf16_t* out;                 // [rows, hq, dh] (n_splits == 1)
    float* o_part;               // [n_splits, rows, hq, dh]
    float* ml_part;              // [n_splits, rows, hq, 2]
    int rows;
};

template <int DH>
struct AttnShape {
    static constexpr int KROWB = DH * 2;             // bytes per K row
    static constexpr int KCH = DH / 8;               // 16-byte chunks per K row
    static constexpr int KBYTES = KT * KROWB;
    static constexpr int VROWB = KT * 2;             // bytes per V^T row (one tile's keys)
    static constexpr int VCH = KT / 8;
    static constexpr int VBYTES = DH * VROWB;
    static constexpr int STAGE = KBYTES + VBYTES;
    static constexpr int KLPT = KBYTES / 4096;       // K loads per thread per stage (1 KB per wave-load)
    static constexpr int LPT = STAGE / 4096;         // all loads per thread per stage
    static constexpr int NS = DH / 32;               // MFMA k-steps over dh
    static constexpr int ND = DH / 16;               // dh sub-tiles of O^T
    static_assert(KBYTES % 4096 == 0 && VBYTES % 4096 == 0, "whole wave-loads per operand");
};

// Tile-relative key of row i (0..15) of 16-key score block u (0..3): lane group
// g holds rows 4g..4g+3 of every block, i.e. keys 32*(u/2) + 8g + 4*(u%2) + v,
// so blocks 2h and 2h+1 together give it keys 32h + 8g .. 32h + 8g + 7.
__device__ __forceinline__ int key_of(int u, int i) {
    return 32 * (u >> 1) + 8 * (i >> 2) + 4 * (u & 1) + (i & 3);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int DH>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs a) {
    using S = AttnShape<DH>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * S::STAGE];

    int b = blockIdx.x;
    const int split = b % a.n_splits; b /= a.n_splits;
    const int qblk = b % a.n_qblocks; b /= a.n_qblocks;
    const int kvh = b % a.hkv; b /= a.hkv;
    const int sq = b;
    const int tid = threadIdx.x, lane = tid % WAVE;
    const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int g = lane / 16, li = lane % 16;
    const int per = a.seqs.per_seq;
    const int T = a.seqs.T[sq];
    const int n_keys = T + per;

    // this lane's two query rows (one per 16-row block)
    const int nq = per * a.group;
    bf16x8 qf[2][S::NS];
    int qpos[2], qh[2];
    long orow[2];
    bool qok[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int qr = qblk * QB + wave * QW + qb * 16 + li;
        qok[qb] = qr < nq;
        const int qi = qok[qb] ? qr / a.group : 0;
        qh[qb] = kvh * a.group + (qok[qb] ? qr % a.group : 0);
        qpos[qb] = T + qi;
        orow[qb] = (long)sq * per + qi;
#pragma unroll
        for (int s = 0; s < S::NS; ++s)
            qf[qb][s] = qok[qb] ? *(const bf16x8*)(a.q + (orow[qb] * a.hq + qh[qb]) * DH + 32 * s + 8 * g)
                                : bf16x8{};
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
    // I = j*4 + wave; K rows first (row, swizzled chunk), then V^T rows (dh, chunk).
    int lrow[S::LPT], lchunk[S::LPT];
#pragma unroll
    for (int j = 0; j < S::LPT; ++j) {
        const int off = (j * 4 + wave) * 1024 + lane * 16;
        if (j < S::KLPT) {
            const int R = off / S::KROWB, p = (off % S::KROWB) / 16;
            lrow[j] = R;
            lchunk[j] = p ^ (R % S::KCH);
        } else {
            const int o = off - S::KBYTES;
            const int d = o / S::VROWB, p = (o % S::VROWB) / 16;
            lrow[j] = d;
            lchunk[j] = p ^ (d % S::VCH);
        }
    }
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
                const int key = k0 + lrow[j];
                src = kb.k + (long)(key < kend ? lrow[j] : 0) * DH + lchunk[j] * 8;
            } else {
                const int kc = k0 + 8 * lchunk[j];
                src = kb.vt + (long)lrow[j] * kb.vstride + (kc < kend ? 8 * lchunk[j] : 0);
            }
            __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(st + (j * 4 + wave) * 1024), 16, 0, 0);
        }
    };
    // V^T slots of keys >= kend in the tile: zero (after this lane's own loads landed)
    auto zero_tail = [&](int tile, int slot) {
        const int k0 = tile * KT;
        if (k0 + KT <= kend) return;
        uint8_t* st = smem + slot * S::STAGE;
#pragma unroll
        for (int j = S::KLPT; j < S::LPT; ++j) {
            const int nv = kend - (k0 + 8 * lchunk[j]);
            if (nv < 8) {
                bf16_t* dst = (bf16_t*)(st + (j * 4 + wave) * 1024 + lane * 16);
                for (int e = max(nv, 0); e < 8; ++e) dst[e] = 0;
            }
        }
    };

    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    f32x4 o[2][S::ND];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int d = 0; d < S::ND; ++d) o[qb][d] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (t0 < t1) issue(t0, 0);
    for (int t = t0; t < t1; ++t) {
        const int slot = (t - t0) & 1;
        if (t + 1 < t1) {
            if (t > t0) stage_barrier();       // every wave is done reading the other slot
            issue(t + 1, slot ^ 1);
            wait_vm<S::LPT>();
        } else {
            wait_vm<0>();
        }
        zero_tail(t, slot);
        stage_barrier();

        const uint8_t* ks = smem + slot * S::STAGE;
        const uint8_t* vs = ks + S::KBYTES;
        const int k0 = t * KT;
        // S^T blocks: 4 x 16 keys, for both query blocks
        f32x4 sc[2][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sc[0][u] = f32x4{0.f, 0.f, 0.f, 0.f};
            sc[1][u] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int R = key_of(u, li);
#pragma unroll
            for (int s = 0; s < S::NS; ++s) {
                const int c = 4 * s + g;
                const bf16x8 kf = *(const bf16x8*)(ks + R * S::KROWB + ((c ^ (R % S::KCH)) << 4));
                sc[0][u] = mfma_bf16(kf, qf[0][s], sc[0][u]);
                sc[1][u] = mfma_bf16(kf, qf[1][s], sc[1][u]);
            }
        }
        // mask, online softmax (per query = per lane column), P = hi + lo
        const bool full = k0 + KT <= kend && !(a.causal && k0 + KT - 1 > wave_pos0);
        bf16x8 ph[2][2], pl[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mt = -INFINITY;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    if (!full) {
                        const int key = k0 + key_of(u, 4 * g + v);
                        if (key >= kend || (a.causal && key > qpos[qb])) sc[qb][u][v] = -INFINITY;
                    }
                    mt = fmaxf(mt, sc[qb][u][v]);
                }
            mt = fmaxf(mt, __shfl_xor(mt, 16, WAVE));
            mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE));
            const float m_new = fmaxf(m_run[qb], mt * a.scale_log2);
            const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run[qb] - m_new);
            m_run[qb] = m_new;
            l_run[qb] *= alpha;
#pragma unroll
            for (int d = 0; d < S::ND; ++d) o[qb][d] *= alpha;
            float p[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    p[u][v] = (m_new == -INFINITY) ? 0.f : exp2f(fmaf(sc[qb][u][v], a.scale_log2, -m_new));
                    l_run[qb] += p[u][v];
                }
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const __bf16 a0 = (__bf16)p[2 * h2][v], a1 = (__bf16)p[2 * h2 + 1][v];
                    ph[qb][h2][v] = a0;
                    ph[qb][h2][4 + v] = a1;
                    pl[qb][h2][v] = (__bf16)(p[2 * h2][v] - (float)a0);
                    pl[qb][h2][4 + v] = (__bf16)(p[2 * h2 + 1][v] - (float)a1);
                }
            }
        }
        // O^T += V^T P^T: per dh sub-tile, two 32-key MFMA steps
#pragma unroll
        for (int d = 0; d < S::ND; ++d) {
            const int row = d * 16 + li;
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int c = 4 * h2 + g;
                const bf16x8 vf = *(const bf16x8*)(vs + row * S::VROWB + ((c ^ (row % S::VCH)) << 4));
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    o[qb][d] = mfma_bf16(vf, ph[qb][h2], o[qb][d]);
                    o[qb][d] = mfma_bf16(vf, pl[qb][h2], o[qb][d]);
                }
            }
        }
    }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        // row sum across the 4 lane groups holding this query
        float l = l_run[qb];
        l += __shfl_xor(l, 16, WAVE);
        l += __shfl_xor(l, 32, WAVE);
        if (!qok[qb]) continue;
        const long obase = (orow[qb] * a.hq + qh[qb]) * DH;
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
                float* ml = a.ml_part + ((long)split * a.rows * a.hq + orow[qb] * a.hq + qh[qb]) * 2;
                ml[0] = m_run[qb];
                ml[1] = l;
            }
        }
    }
}

// Merge split partials: O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j, in
// split order.  One thread per 4 consecutive dh elements of a (row, head).
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* o_part, const float* ml_part, int n_splits,
                                                          long pairs, int dh, bf16_t* out) {
    const int tpp = dh / 4;                       // threads per (row, head)
    const long t = (long)blockIdx.x * 256 + threadIdx.x;
    const long rh = t / tpp;
    if (rh >= pairs) return;
    const int c = (int)(t % tpp) * 4;
    float M = -INFINITY;
    for (int j = 0; j < n_splits; ++j) M = fmaxf(M, ml_part[(j * pairs + rh) * 2]);
    float L = 0.f;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < n_splits; ++j) {
        const float m = ml_part[(j * pairs + rh) * 2];
        if (m == -INFINITY) continue;
        const float w = exp2f(m - M);
        L += w * ml_part[(j * pairs + rh) * 2 + 1];
        acc += w * *(const f32x4*)(o_part + (j * pairs + rh) * dh + c);
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
// partial buffers); each split keeps at least 4 key tiles; aim for about
// SPLIT_TARGET workgroups (two per CU).
constexpr int SPLIT_ROWS = 4096;
constexpr int SPLIT_TARGET = 512;

static int choose_splits(int base_blocks, int ntiles, int rows) {
    int s = (SPLIT_TARGET + base_blocks - 1) / base_blocks;
    s = min(s, max(1, ntiles / 4));
    s = min(s, max(1, SPLIT_ROWS / rows));
    return max(1, min(s, MAX_SPLITS));
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
    a.n_qblocks = (seqs.per_seq * a.group + QB - 1) / QB;
    int max_keys = 0;
    for (int i = 0; i < seqs.n; ++i) max_keys = max(max_keys, seqs.T[i] + seqs.per_seq);
    const int ntiles = (max_keys + KT - 1) / KT;
    const int base = seqs.n * hkv * a.n_qblocks;
    a.n_splits = causal ? 1 : choose_splits(base, ntiles, rows);
    a.tiles_per_split = (ntiles + a.n_splits - 1) / a.n_splits;
    a.n_splits = (ntiles + a.tiles_per_split - 1) / a.tiles_per_split;
    if (a.n_splits < 1) a.n_splits = 1;
    a.scale_log2 = LOG2E / sqrtf((float)dh);
    a.out = (bf16_t*)out;
    a.o_part = w.o_part;
    a.ml_part = w.ml_part;
    a.rows = rows;
    const dim3 grid(base * a.n_splits);
    if (dh == 128) launch(attn_bf16_kernel<128>, grid, dim3(256), 0, st, a);
    else if (dh == 64) launch(attn_bf16_kernel<64>, grid, dim3(256), 0, st, a);
    else launch(attn_bf16_kernel<32>, grid, dim3(256), 0, st, a);
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
