// Row-wise kernels of the transformer block: embedding gather, RMSNorm with the
// residual update and the GEMM-operand casts fused in (bf16, and per-token E4M3
// for fp8 models), per-row E4M3 quantisation, and rotary embedding fused with
// the K/V cache write.  All are HBM/latency bound: one wave per token row where
// a row fits the wave's registers, 16-byte accesses, fixed-order reductions.
//
// Split-K consumers.  A weight-streaming GEMM that split its K range leaves
// fp32 partials [splits][rows][cols]; the kernel that reads its result next
// sums them in split order (applying the fp8 scales): RMSNorm adds the O- and
// down-projection partials into the residual stream, RoPE sums the QKV
// partials.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "kvcache.h"

namespace dlm {

constexpr int NT = 256;

// Partials of GEMM output rows: the direct fp32 output (splits == 1, already
// scaled) or split-K partials [splits][rows][cols], summed in split order.
__device__ __forceinline__ f32x4 partial_sum4(const Partials& p, int row, int col, int ncols) {
    const long off = (long)row * ncols + col;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.splits; ++s) v += *(const f32x4*)(p.p + s * p.stride + off);
    if (p.a_scale) {
        const float sa = p.a_scale[row];
        const f32x4 sb = *(const f32x4*)(p.b_scale + col);
        v = v * sa * sb;
    }
    return v;
}

// ------------------------------------------------------------------ embed --

__global__ __launch_bounds__(NT) void embed_kernel(IdSource ids, const void* table, int dtype, int d,
                                                    int vocab, int mask_id, int check_mask, float* x,
                                                    int* err) {
    const int r = blockIdx.x;
    int id = ids.flat ? ids.flat[r] : ids.canvas[r / ids.per_seq][r % ids.per_seq];
    if (threadIdx.x == 0) {
        if (id < 0 || id >= vocab) atomicOr(err, DEVERR_TOKEN_RANGE);
        if (check_mask && id == mask_id) atomicOr(err, DEVERR_MASK_APPEND);
    }
    if (id < 0 || id >= vocab) id = 0;
    float* xr = x + (long)r * d;
    if (dtype == DT_F32) {
        const float* t = (const float*)table + (long)id * d;
        for (int c = threadIdx.x; c < d; c += NT) xr[c] = t[c];
    } else {
        const bf16_t* t = (const bf16_t*)table + (long)id * d;
        for (int c = threadIdx.x; c < d; c += NT) xr[c] = bf16_to_f32(t[c]);
    }
}

void embed(const IdSource& ids, int rows, const void* table, int dtype, int d, int vocab,
           int mask_id, bool check_mask, float* x, int* err, hipStream_t st) {
    if (rows <= 0) return;
    launch(embed_kernel, dim3(rows), dim3(NT), 0, st, ids, table, dtype, d, vocab, mask_id, (int)check_mask, x,
           err);
}

// ---------------------------------------------------------------- rmsnorm --
// One row per workgroup of four waves; thread t holds the float4 chunks t,
// t + 256, ... of the row (d <= 4 * 256 * MAXC).  x += residual partials and
// the MoE layer's routed experts (if any), then h = x / sqrt(mean(x^2) + eps) * g.

constexpr int RN_T = 256;    // threads per row (4 waves)
constexpr int MAXC = 4;       // float4 per thread: d <= 4 * RN_T * MAXC
constexpr int RN_SG = 8;      // routed-expert rows loaded together (top-8 in one round trip)

// MC: float4 chunks per thread (MAXC, or 3 when d <= 3072: fewer registers
// for the slot rows in flight).  YB: the routed experts' rows are bf16 (held
// as raw 8-byte groups until use, half the registers of fp32 rows).
template <int MC, bool YB>
__global__ __launch_bounds__(RN_T) void rmsnorm_kernel(float* x, Partials res, MoeGather moe, const float* g, int rows,
                                                        int d, float eps, float* hf, bf16_t* hb, fp8_t* hq, float* hs) {
    constexpr int MAXC = MC;
    __shared__ float red[RN_T / WAVE];
    const int lane = threadIdx.x;      // thread of the row (4 waves per row)
    const int r = blockIdx.x;
    if (r >= rows) return;
    const int nc = d / 4;
    const bool out = hf || hb;
    float* xr = x + (long)r * d;
    f32x4 v[MAXC], gg[MAXC];
    float ss = 0.f;
    // every load of the row (x, pending partials, gains) is issued before the first use
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int c = lane + RN_T * k;
        if (c < nc) {
            v[k] = *(const f32x4*)(xr + 4 * c);
            if (out) gg[k] = *(const f32x4*)(g + 4 * c);
        }
    }
    if (res.p || moe.y) {
        // split by split (fixed order); each split's loads of the whole row
        // are issued together, so a row costs one round trip per split
        f32x4 acc[MAXC];
#pragma unroll
        for (int k = 0; k < MAXC; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; res.p && sp < res.splits; ++sp) {
            const float* pr = res.p + sp * res.stride + (long)r * d;
            f32x4 t[MAXC];
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int c = lane + RN_T * k;
                if (c < nc) t[k] = *(const f32x4*)(pr + 4 * c);
            }
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int c = lane + RN_T * k;
                if (c < nc) acc[k] += t[k];
            }
        }
        if (res.p && res.a_scale) {
            const float sa = res.a_scale[r];
#pragma unroll
            for (int k = 0; k < MAXC; ++k) {
                const int c = lane + RN_T * k;
                if (c < nc) acc[k] = acc[k] * sa * *(const f32x4*)(res.b_scale + 4 * c);
            }
        }
        // routed experts, slot by slot in selection order; the rows of RN_SG
        // slots are loaded together (one round trip per RN_SG slots)
        for (int s0 = 0; moe.y && s0 < moe.k; s0 += RN_SG) {
            typedef std::conditional_t<YB, uint2, f32x4> yrow_t;
            yrow_t yv[RN_SG][MAXC];
            float ws[RN_SG];
#pragma unroll
            for (int j = 0; j < RN_SG; ++j) {
                if (s0 + j >= moe.k) break;
                const long a = (long)r * moe.k + s0 + j;
                ws[j] = moe.w[a];
                const long yo = (long)moe.inv[a] * d;
#pragma unroll
                for (int k = 0; k < MAXC; ++k) {
                    const int c = lane + RN_T * k;
                    if (c < nc) {
                        if constexpr (YB) yv[j][k] = *(const uint2*)((const bf16_t*)moe.y + yo + 4 * c);
                        else yv[j][k] = *(const f32x4*)((const float*)moe.y + yo + 4 * c);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < RN_SG; ++j) {
                if (s0 + j >= moe.k) break;
#pragma unroll
                for (int k = 0; k < MAXC; ++k) {
                    const int c = lane + RN_T * k;
                    if (c < nc) {
                        if constexpr (YB) {
                            const uint2 u = yv[j][k];
                            const f32x4 y = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                                  __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
                            acc[k] += ws[j] * y;
                        } else {
                            acc[k] += ws[j] * yv[j][k];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int c = lane + RN_T * k;
            if (c < nc) v[k] += acc[k];
        }
#pragma unroll
        for (int k = 0; k < MAXC; ++k) {
            const int c = lane + RN_T * k;
            if (c < nc) *(f32x4*)(xr + 4 * c) = v[k];
        }
    }
    if (!out) return;                              // residual update only
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int c = lane + RN_T * k;
        if (c < nc) ss += v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
    }
    // row sums across the four waves, added in wave order
    ss = wave_sum(ss);
    if (lane % WAVE == 0) red[lane / WAVE] = ss;
    __syncthreads();
    ss = (red[0] + red[1]) + (red[2] + red[3]);
    const float den = sqrtf(ss / (float)d + eps);
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int c = lane + RN_T * k;
        if (c < nc) {
            f32x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = v[k][e] / den * gg[k][e];
            if (hf) *(f32x4*)(hf + (long)r * d + 4 * c) = h;
            if (hb) {
                uint64_t packed = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bf16_t b = f32_to_bf16(h[e]);
                    packed |= (uint64_t)b << (16 * e);
                    v[k][e] = bf16_to_f32(b);          // keep the stored value for quantisation
                    amax = fmaxf(amax, fabsf(v[k][e]));
                }
                *(uint64_t*)(hb + (long)r * d + 4 * c) = packed;
            }
        }
    }
    if (!hq) return;
    amax = wave_max(amax);
    __syncthreads();                   // every wave has read red[] above
    if (lane % WAVE == 0) red[lane / WAVE] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int c = lane + RN_T * k;
        if (c < nc) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) packed |= (uint32_t)f32_to_e4m3(v[k][e] / sc) << (8 * e);
            *(uint32_t*)(hq + (long)r * d + 4 * c) = packed;
        }
    }
    if (lane == 0) hs[r] = sc;
}

void rmsnorm(float* x, const Partials& res, const MoeGather& moe, const float* g, int rows, int d, float eps,
             float* hf, uint16_t* hb, uint8_t* hq, float* hs, hipStream_t st) {
    if (rows <= 0) return;
    const bool yb = moe.y && moe.y_bf16;
    if (d <= 4 * RN_T * 3) {
        if (yb) launch(rmsnorm_kernel<3, true>, dim3(rows), dim3(RN_T), 0, st, x, res, moe, g, rows, d, eps, hf, hb, hq, hs);
        else launch(rmsnorm_kernel<3, false>, dim3(rows), dim3(RN_T), 0, st, x, res, moe, g, rows, d, eps, hf, hb, hq, hs);
    } else {
        if (yb) launch(rmsnorm_kernel<MAXC, true>, dim3(rows), dim3(RN_T), 0, st, x, res, moe, g, rows, d, eps, hf, hb, hq, hs);
        else launch(rmsnorm_kernel<MAXC, false>, dim3(rows), dim3(RN_T), 0, st, x, res, moe, g, rows, d, eps, hf, hb, hq, hs);
    }
}

int rmsnorm_max_dim() { return 4 * RN_T * MAXC; }

// ------------------------------------------------------------- quant_rows --

__device__ __forceinline__ float block_max(float v, float* red) {
    v = wave_max(v);
    const int w = threadIdx.x / WAVE;
    __syncthreads();
    if (threadIdx.x % WAVE == 0) red[w] = v;
    __syncthreads();
    float s = red[0];
#pragma unroll
    for (int i = 1; i < NT / WAVE; ++i) s = fmaxf(s, red[i]);
    return s;
}

__global__ __launch_bounds__(NT) void quant_rows_kernel(const bf16_t* x, int d, fp8_t* q, float* s) {
    __shared__ float red[NT / WAVE];
    const long r = blockIdx.x;
    float amax = 0.f;
    for (int c = threadIdx.x; c < d; c += NT) amax = fmaxf(amax, fabsf(bf16_to_f32(x[r * d + c])));
    amax = block_max(amax, red);
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
    for (int c = threadIdx.x; c < d; c += NT) q[r * d + c] = f32_to_e4m3(bf16_to_f32(x[r * d + c]) / sc);
    if (threadIdx.x == 0) s[r] = sc;
}

// d % 8 == 0 and d <= 8 * NT * QV: each thread keeps its 8-element chunks in
// registers between the row maximum and the conversion (one 16-byte load and
// one 8-byte store per chunk).
constexpr int QV = 4;
__global__ __launch_bounds__(NT) void quant_rows_vec_kernel(const bf16_t* x, int d, fp8_t* q, float* s) {
    __shared__ float red[NT / WAVE];
    const long r = blockIdx.x;
    const int nch = d / 8;
    uint4 raw[QV];
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < QV; ++k) {
        const int c = threadIdx.x + NT * k;
        if (c < nch) {
            raw[k] = *(const uint4*)(x + r * d + 8 * c);
            const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xffff0000u))));
        }
    }
    amax = block_max(amax, red);
    const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < QV; ++k) {
        const int c = threadIdx.x + NT * k;
        if (c < nch) {
            const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                lo |= (uint32_t)f32_to_e4m3(__uint_as_float(w[e] << 16) / sc) << (16 * e);
                lo |= (uint32_t)f32_to_e4m3(__uint_as_float(w[e] & 0xffff0000u) / sc) << (16 * e + 8);
                hi |= (uint32_t)f32_to_e4m3(__uint_as_float(w[2 + e] << 16) / sc) << (16 * e);
                hi |= (uint32_t)f32_to_e4m3(__uint_as_float(w[2 + e] & 0xffff0000u) / sc) << (16 * e + 8);
            }
            *(uint2*)(q + r * d + 8 * c) = uint2{lo, hi};
        }
    }
    if (threadIdx.x == 0) s[r] = sc;
}

void quant_rows(const uint16_t* x, int rows, int d, uint8_t* q, float* s, hipStream_t st) {
    if (rows <= 0) return;
    if (d % 8 == 0 && d <= 8 * NT * QV)
        launch(quant_rows_vec_kernel, dim3(rows), dim3(NT), 0, st, (const bf16_t*)x, d, q, s);
    else
        launch(quant_rows_kernel, dim3(rows), dim3(NT), 0, st, (const bf16_t*)x, d, q, s);
}

// ---------------------------------------------------------------- rope_kv --
// Rotate-half rotary embedding: for i < dh/2 the pair (v[i], v[i + dh/2]) is
// rotated by pos * base^(-2i/dh).  The angle and its sine/cosine are formed in
// double precision (positions reach several thousand), then applied in fp32.
//
// Cache layout (kvcache.h): per (layer, KV head) K as rows [token][dh] and V
// transposed [dh][token], contiguous or in 64-token pages, so the attention
// kernel's P V operand reads consecutive keys.  Blocks [0, rows) rotate Q and
// K of one token row;
// the blocks after them each transpose V of up to 64 rows of one KV head
// through LDS, so every wave writes 64 consecutive positions of one dh row.
constexpr int VT_ROWS = 64;                // rows per V^T block
constexpr int VT_COLS = 32;                // value dimensions per V^T block

template <bool F32>
__global__ __launch_bounds__(NT) void rope_kv_kernel(Partials qkv, SeqTab seqs, int rows, int layer, int hq,
                                                      int hkv, int dh, float base, void* q_out) {
    typedef typename std::conditional<F32, float, bf16_t>::type T;
    constexpr int PITCH = VT_COLS + (F32 ? 1 : 2);   // conflict-free column reads
    constexpr int PER_T = VT_ROWS * VT_COLS / NT;    // elements per thread
    __shared__ T tile[VT_ROWS * PITCH];
    const int ncols = (hq + 2 * hkv) * dh;
    if ((int)blockIdx.x >= rows) {
        const int nslice = dh / VT_COLS;
        int vb = blockIdx.x - rows;
        const int sl = vb % nslice; vb /= nslice;
        const int kh = vb % hkv, r0 = (vb / hkv) * VT_ROWS;
        const int nr = min(VT_ROWS, rows - r0);
        const int col0 = (hq + hkv + kh) * dh + sl * VT_COLS;
        float val[PER_T];
#pragma unroll
        for (int i = 0; i < PER_T; ++i) val[i] = 0.f;
        for (int sp = 0; sp < qkv.splits; ++sp) {
            const float* pr = qkv.p + sp * qkv.stride + (long)r0 * ncols + col0;
            float t[PER_T];
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int e = threadIdx.x + NT * i, rr = e / VT_COLS, d = e % VT_COLS;
                if (rr < nr) t[i] = pr[(long)rr * ncols + d];
            }
#pragma unroll
            for (int i = 0; i < PER_T; ++i) val[i] += t[i];
        }
        if (qkv.a_scale) {
#pragma unroll
            for (int i = 0; i < PER_T; ++i) {
                const int e = threadIdx.x + NT * i, rr = e / VT_COLS, d = e % VT_COLS;
                if (rr < nr) val[i] *= qkv.a_scale[r0 + rr] * qkv.b_scale[col0 + d];
            }
        }
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int e = threadIdx.x + NT * i, rr = e / VT_COLS, d = e % VT_COLS;
            if constexpr (F32) tile[rr * PITCH + d] = val[i];
            else tile[rr * PITCH + d] = f32_to_bf16(val[i]);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER_T; ++i) {
            const int e = threadIdx.x + NT * i, d = e / VT_ROWS, rr = e % VT_ROWS;
            if (rr >= nr) continue;
            const int r = r0 + rr, s = r / seqs.per_seq;
            const int pos = seqs.T[s] + r % seqs.per_seq;
            const KVBlock<T> b = kv_block<T>(seqs, s, layer, hkv, kh, dh, pos / KV_PAGE);
            b.vt[(long)(sl * VT_COLS + d) * b.vstride + pos % KV_PAGE] = tile[rr * PITCH + d];
        }
        return;
    }
    const int r = blockIdx.x;
    const int s = r / seqs.per_seq, i = r % seqs.per_seq;
    const int pos = seqs.T[s] + i;
    const int half = dh / 2;
    const int j = threadIdx.x % half;        // pair index
    const int hg = threadIdx.x / half;       // head lane group
    const int ngroups = NT / half;
    const int nh = hq + hkv;                 // rotated heads: Q, then K
    // every head's pair is loaded before the first is used (one round trip)
    constexpr int MAXIT = 16;                // ceil(nh / ngroups) <= 16 for the supported shapes
    float av[MAXIT], bv[MAXIT];
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) av[it] = bv[it] = 0.f;
    for (int sp = 0; sp < qkv.splits; ++sp) {
        const float* pr = qkv.p + sp * qkv.stride + (long)r * ncols + j;
        float ta[MAXIT], tb[MAXIT];
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
            const int h = hg + it * ngroups;
            if (h < nh) {
                ta[it] = pr[h * dh];
                tb[it] = pr[h * dh + half];
            }
        }
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
            av[it] += ta[it];
            bv[it] += tb[it];
        }
    }
    if (qkv.a_scale) {
        const float sa = qkv.a_scale[r];
#pragma unroll
        for (int it = 0; it < MAXIT; ++it) {
            const int h = hg + it * ngroups;
            if (h < nh) {
                av[it] *= sa * qkv.b_scale[h * dh + j];
                bv[it] *= sa * qkv.b_scale[h * dh + j + half];
            }
        }
    }
    const double theta = pow((double)base, -2.0 * (double)j / (double)dh);
    double sd, cd;
    sincos((double)pos * theta, &sd, &cd);
    const float sn = (float)sd, cs = (float)cd;
#pragma unroll
    for (int it = 0; it < MAXIT; ++it) {
        const int h = hg + it * ngroups;
        if (h >= nh) continue;
        const float a = av[it], b = bv[it];
        const float ra = a * cs - b * sn;
        const float rb = a * sn + b * cs;
        T* dst;
        if (h < hq) {
            dst = (T*)q_out + ((long)r * hq + h) * dh;
        } else {
            dst = kv_block<T>(seqs, s, layer, hkv, h - hq, dh, pos / KV_PAGE).k + (long)(pos % KV_PAGE) * dh;
        }
        if constexpr (F32) {
            dst[j] = ra;
            dst[j + half] = rb;
        } else {
            dst[j] = f32_to_bf16(ra);
            dst[j + half] = f32_to_bf16(rb);
        }
    }
}

void rope_kv(const Partials& qkv, int rows, const SeqTab& seqs, int layer, int n_layers, int hq, int hkv, int dh,
             float base, bool f32, void* q_out, hipStream_t st) {
    (void)n_layers;
    if (rows <= 0) return;
    const dim3 grid(rows + (rows + VT_ROWS - 1) / VT_ROWS * hkv * (dh / VT_COLS));
    if (f32)
        launch(rope_kv_kernel<true>, grid, dim3(NT), 0, st, qkv, seqs, rows, layer, hq, hkv, dh, base, q_out);
    else
        launch(rope_kv_kernel<false>, grid, dim3(NT), 0, st, qkv, seqs, rows, layer, hq, hkv, dh, base, q_out);
}

}  // namespace dlm
