// Attention over the KV cache for gfx950.
//
// Denoising ("block") mode: every canvas query sees every cached key [0, T) and
// every canvas key [T, T + C) -- bidirectional inside the canvas, full to the
// prefix.  Prefill ("causal") mode: the query at position p sees keys [0, p].
// Grouped-query attention: query head h reads KV head h / (Hq / Hkv).
//
// bf16 kernel (flash-style, online softmax in fp32):
//   * A workgroup owns one KV head of one request and 64 "query rows" (pairs of
//     canvas position and query head of that KV head's group), so every query
//     of the group shares each K/V tile staged in LDS.
//   * Scores are computed transposed, S^T = K Q^T, with 16x16x32 bf16 MFMAs:
//     the output puts one query per lane column, so the row statistics of the
//     online softmax are per-lane scalars, and the probabilities P^T are
//     already laid out as the B operand of O^T = V^T P^T (the K order inside
//     one MFMA is a permutation shared by both operands).  V is staged
//     transposed in LDS so the A operand reads are 8-byte vectors.  P is fed
//     as two bf16 terms (hi + lo), so P V carries fp32-level precision.
//   * Long key ranges are split across workgroups (split-KV); partial (max,
//     sum, unnormalised O) are merged by a second kernel in fixed split order.
// fp32 kernel (fp32 models): one thread per (query, head), online softmax,
// fp32 throughout.
#include "common.h"
#include "kernels.h"

namespace dlm {

constexpr int QB = 64;          // query rows per workgroup
constexpr int KT = 64;          // keys per tile
constexpr int MAX_SPLITS = 16;
constexpr float LOG2E = 1.4426950408889634f;

struct AttnArgs {
    const bf16_t* q;            // [rows, hq, dh]
    SeqTab seqs;
    int layer, hq, hkv, group;
    int causal;
    int n_qblocks;              // per (request, kv head)
    int n_splits;
    int tiles_per_split;
    float scale_log2;           // dh^-1/2 * log2(e)
    bf16_t* out;                // [rows, hq, dh] (n_splits == 1)
    float* o_part;              // [n_splits, rows, hq, dh]
    float* ml_part;             // [n_splits, rows, hq, 2]
    int rows;
};

template <int DH>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnArgs a) {
    constexpr int KROW = DH * 2 + 16;              // bytes per K row in LDS
    constexpr int VROW = KT * 2 + 16;              // bytes per V^T row in LDS
    constexpr int NS = DH / 32;                    // MFMA k-steps over dh
    constexpr int ND = DH / 16;                    // dh sub-tiles of O^T
    __shared__ __attribute__((aligned(16))) uint8_t ks[KT * KROW];
    __shared__ __attribute__((aligned(16))) uint8_t vt[DH * VROW];

    int b = blockIdx.x;
    const int split = b % a.n_splits; b /= a.n_splits;
    const int qblk = b % a.n_qblocks; b /= a.n_qblocks;
    const int kvh = b % a.hkv; b /= a.hkv;
    const int sq = b;
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int g4 = lane / 16;
    const int per = a.seqs.per_seq;
    const int T = a.seqs.T[sq];
    const int n_keys = T + per;
    const long cap = a.seqs.cap[sq];
    const bf16_t* kbase = (const bf16_t*)a.seqs.kv[sq] + (((long)a.layer * 2 + 0) * a.hkv + kvh) * cap * DH;
    const bf16_t* vbase = (const bf16_t*)a.seqs.kv[sq] + (((long)a.layer * 2 + 1) * a.hkv + kvh) * cap * DH;

    // this lane's query row
    const int nq = per * a.group;
    const int qr = qblk * QB + wave * 16 + lane % 16;
    const bool qok = qr < nq;
    const int qi = qok ? qr / a.group : 0;
    const int qh = kvh * a.group + (qok ? qr % a.group : 0);
    const int qpos = T + qi;
    const long orow = (long)sq * per + qi;

    bf16x8 qf[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (qok) qf[s] = *(const bf16x8*)(a.q + (orow * a.hq + qh) * DH + 32 * s + 8 * g4);
        else qf[s] = bf16x8{};
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

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[ND];
#pragma unroll
    for (int d = 0; d < ND; ++d) o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging assignment
    constexpr int KCH = KT * DH / 8;               // 16-byte chunks of a K tile
    constexpr int KPT = (KCH + 255) / 256;
    constexpr int VQ = (KT / 4) * (DH / 8);         // (key quad, dh chunk) pairs of a V tile
    constexpr int VPT = (VQ + 255) / 256;
    uint4 rk[KPT], rv[VPT][4];

    auto gload = [&](int tile) {
        const int k0 = tile * KT;
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int c = tid + 256 * j;
            const int key = k0 + c / (DH / 8);
            rk[j] = (c < KCH && key < kend) ? *(const uint4*)(kbase + (long)key * DH + (c % (DH / 8)) * 8)
                                             : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int w = tid + 256 * j;
            const int quad = w / (DH / 8), dc = w % (DH / 8);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int key = k0 + quad * 4 + kk;
                rv[j][kk] = (w < VQ && key < kend) ? *(const uint4*)(vbase + (long)key * DH + dc * 8)
                                                    : uint4{0, 0, 0, 0};
            }
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int c = tid + 256 * j;
            if (c < KCH) *(uint4*)(ks + (c / (DH / 8)) * KROW + (c % (DH / 8)) * 16) = rk[j];
        }
#pragma unroll
        for (int j = 0; j < VPT; ++j) {
            const int w = tid + 256 * j;
            if (w >= VQ) continue;
            const int quad = w / (DH / 8), dc = w % (DH / 8);
            const uint16_t* e0 = (const uint16_t*)&rv[j][0];
            const uint16_t* e1 = (const uint16_t*)&rv[j][1];
            const uint16_t* e2 = (const uint16_t*)&rv[j][2];
            const uint16_t* e3 = (const uint16_t*)&rv[j][3];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint64_t packed = (uint64_t)e0[e] | ((uint64_t)e1[e] << 16) | ((uint64_t)e2[e] << 32) |
                                        ((uint64_t)e3[e] << 48);
                *(uint64_t*)(vt + (dc * 8 + e) * VROW + quad * 8) = packed;
            }
        }
    };

    if (t0 < t1) gload(t0);
    for (int t = t0; t < t1; ++t) {
        __syncthreads();                  // previous tile's LDS reads are done
        sstore();
        __syncthreads();
        if (t + 1 < t1) gload(t + 1);
        const int k0 = t * KT;
        // S^T tile: 4 key sub-tiles of 16
        f32x4 st[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            st[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bf16x8 kf = *(const bf16x8*)(ks + (u * 16 + lane % 16) * KROW + (32 * s + 8 * g4) * 2);
                st[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], st[u], 0, 0, 0);
            }
        }
        // scale, mask, online softmax (per query = per lane column)
        float mt = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int key = k0 + u * 16 + 4 * g4 + v;
                float sc = st[u][v] * a.scale_log2;
                if (key >= kend || (a.causal && key > qpos) || !qok) sc = -INFINITY;
                st[u][v] = sc;
                mt = fmaxf(mt, sc);
            }
        mt = fmaxf(mt, __shfl_xor(mt, 16, WAVE));
        mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < ND; ++d) o[d] *= alpha;
        // P = hi + lo, both bf16: the product with V is then exact to ~2^-16
        // relative instead of bf16's 2^-9 (two MFMAs per step).
        bf16_t pb[4][4], pl[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float p = (st[u][v] == -INFINITY) ? 0.f : exp2f(st[u][v] - m_new);
                l_run += p;
                pb[u][v] = f32_to_bf16(p);
                pl[u][v] = f32_to_bf16(p - bf16_to_f32(pb[u][v]));
            }
        // O^T += V^T P^T over two 32-key MFMA steps
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            bf16x8 pf, pf_lo;
            uint16_t* pu = (uint16_t*)&pf;
            uint16_t* pv = (uint16_t*)&pf_lo;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                pu[v] = pb[2 * h2][v];
                pu[4 + v] = pb[2 * h2 + 1][v];
                pv[v] = pl[2 * h2][v];
                pv[4 + v] = pl[2 * h2 + 1][v];
            }
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const uint8_t* vr = vt + (d * 16 + lane % 16) * VROW;
                const uint64_t lo = *(const uint64_t*)(vr + (32 * h2 + 4 * g4) * 2);
                const uint64_t hi = *(const uint64_t*)(vr + (32 * h2 + 16 + 4 * g4) * 2);
                bf16x8 vf;
                ((uint64_t*)&vf)[0] = lo;
                ((uint64_t*)&vf)[1] = hi;
                o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[d], 0, 0, 0);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf_lo, o[d], 0, 0, 0);
            }
        }
    }
    // row sum across the 4 lane groups holding this query
    l_run += __shfl_xor(l_run, 16, WAVE);
    l_run += __shfl_xor(l_run, 32, WAVE);
    if (!qok) return;
    const long obase = (orow * a.hq + qh) * DH;
    if (a.n_splits == 1) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            uint64_t packed = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) packed |= (uint64_t)f32_to_bf16(o[d][v] * inv) << (16 * v);
            *(uint64_t*)(a.out + obase + d * 16 + 4 * g4) = packed;
        }
    } else {
        float* op = a.o_part + (long)split * a.rows * a.hq * DH + obase;
#pragma unroll
        for (int d = 0; d < ND; ++d) *(f32x4*)(op + d * 16 + 4 * g4) = o[d];
        if (g4 == 0) {
            float* ml = a.ml_part + ((long)split * a.rows * a.hq + orow * a.hq + qh) * 2;
            ml[0] = m_run;
            ml[1] = l_run;
        }
    }
}

// Merge split partials: O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j.
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* o_part, const float* ml_part, int n_splits,
                                                          int rows, int hq, int dh, bf16_t* out) {
    const long rh = blockIdx.x;               // (row, head)
    const long total = (long)rows * hq;
    float M = -INFINITY;
    for (int j = 0; j < n_splits; ++j) M = fmaxf(M, ml_part[(j * total + rh) * 2]);
    float L = 0.f;
    for (int j = 0; j < n_splits; ++j) {
        const float m = ml_part[(j * total + rh) * 2];
        if (m != -INFINITY) L += exp2f(m - M) * ml_part[(j * total + rh) * 2 + 1];
    }
    for (int c = threadIdx.x; c < dh; c += blockDim.x) {
        float acc = 0.f;
        for (int j = 0; j < n_splits; ++j) {
            const float m = ml_part[(j * total + rh) * 2];
            if (m != -INFINITY) acc += exp2f(m - M) * o_part[(j * total + rh) * dh + c];
        }
        out[rh * dh + c] = f32_to_bf16(L > 0.f ? acc / L : 0.f);
    }
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
    const long cap = seqs.cap[sq];
    const float* kb = (const float*)seqs.kv[sq] + (((long)layer * 2 + 0) * hkv + kvh) * cap * DH;
    const float* vb = (const float*)seqs.kv[sq] + (((long)layer * 2 + 1) * hkv + kvh) * cap * DH;
    const int kend = causal ? pos + 1 : T + per;
    float qv[DH], o[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) {
        qv[c] = q[((long)r * hq + h) * DH + c];
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int k = 0; k < kend; ++k) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < DH; ++c) s += qv[c] * kb[(long)k * DH + c];
        s *= scale;
        const float mn = fmaxf(m, s);
        const float al = expf(m - mn);
        const float p = expf(s - mn);
        l = l * al + p;
#pragma unroll
        for (int c = 0; c < DH; ++c) o[c] = o[c] * al + p * vb[(long)k * DH + c];
        m = mn;
    }
#pragma unroll
    for (int c = 0; c < DH; ++c) out[((long)r * hq + h) * DH + c] = o[c] / l;
}

// Split-KV only while splits * rows stays within SPLIT_ROWS (bounds the
// partial buffers); each split keeps at least 4 key tiles.
constexpr int SPLIT_ROWS = 4096;

static int choose_splits(int base_blocks, int ntiles, int rows) {
    int s = (512 + base_blocks - 1) / base_blocks;
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
        launch(attn_merge_kernel, dim3(rows * hq), dim3(128), 0, st, w.o_part, w.ml_part, a.n_splits,
               rows, hq, dh, (bf16_t*)out);
        launch_timer() = t;
    }
}

}  // namespace dlm
