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
#include "common.h"
#include "kernels.h"

namespace dlm {

constexpr int NT = 256;

// Value of output element (row, col) of a GEMM, from its direct fp32 output
// (splits == 1, already scaled) or from its split-K partials.
__device__ __forceinline__ float partial_sum(const Partials& p, int row, int col, int ncols) {
    const long off = (long)row * ncols + col;
    float v = 0.f;
    for (int s = 0; s < p.splits; ++s) v += p.p[s * p.stride + off];
    if (p.a_scale) v *= p.a_scale[row] * p.b_scale[col];
    return v;
}

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
// One wave per row; lane l holds the float4 chunks l, l + 64, ... of the row
// (d <= 4 * 64 * MAXC).  x += residual partials (if any), then
// h = x / sqrt(mean(x^2) + eps) * g.

constexpr int MAXC = 16;

__global__ __launch_bounds__(WAVE) void rmsnorm_kernel(float* x, Partials res, const float* g, int rows, int d,
                                                        float eps, float* hf, bf16_t* hb, fp8_t* hq, float* hs) {
    const int lane = threadIdx.x;
    const int r = blockIdx.x;          // one single-wave workgroup per row: every row on its own CU slot
    if (r >= rows) return;
    const int nc = d / 4;
    float* xr = x + (long)r * d;
    f32x4 v[MAXC];
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int c = lane + WAVE * k;
        if (c < nc) {
            v[k] = *(const f32x4*)(xr + 4 * c);
            if (res.p) {
                v[k] += partial_sum4(res, r, 4 * c, d);
                *(f32x4*)(xr + 4 * c) = v[k];
            }
            ss += v[k][0] * v[k][0] + v[k][1] * v[k][1] + v[k][2] * v[k][2] + v[k][3] * v[k][3];
        }
    }
    if (!hf && !hb) return;                        // residual update only
    const float den = sqrtf(wave_sum(ss) / (float)d + eps);
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int c = lane + WAVE * k;
        if (c < nc) {
            const f32x4 gg = *(const f32x4*)(g + 4 * c);
            f32x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = v[k][e] / den * gg[e];
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
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
#pragma unroll
    for (int k = 0; k < MAXC; ++k) {
        const int c = lane + WAVE * k;
        if (c < nc) {
            uint32_t packed = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) packed |= (uint32_t)f32_to_e4m3(v[k][e] / s) << (8 * e);
            *(uint32_t*)(hq + (long)r * d + 4 * c) = packed;
        }
    }
    if (lane == 0) hs[r] = s;
}

void rmsnorm(float* x, const Partials& res, const float* g, int rows, int d, float eps, float* hf, uint16_t* hb,
             uint8_t* hq, float* hs, hipStream_t st) {
    if (rows <= 0) return;
    launch(rmsnorm_kernel, dim3(rows), dim3(WAVE), 0, st, x, res, g, rows, d, eps, hf, hb, hq, hs);
}

int rmsnorm_max_dim() { return 4 * WAVE * MAXC; }

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

void quant_rows(const uint16_t* x, int rows, int d, uint8_t* q, float* s, hipStream_t st) {
    if (rows <= 0) return;
    launch(quant_rows_kernel, dim3(rows), dim3(NT), 0, st, x, d, q, s);
}

// ---------------------------------------------------------------- rope_kv --
// Rotate-half rotary embedding: for i < dh/2 the pair (v[i], v[i + dh/2]) is
// rotated by pos * base^(-2i/dh).  The angle and its sine/cosine are formed in
// double precision (positions reach several thousand), then applied in fp32.

template <bool F32>
__global__ __launch_bounds__(NT) void rope_kv_kernel(Partials qkv, SeqTab seqs, int layer, int hq, int hkv, int dh,
                                                      float base, void* q_out) {
    const int r = blockIdx.x;
    const int s = r / seqs.per_seq, i = r % seqs.per_seq;
    const int pos = seqs.T[s] + i;
    const int half = dh / 2;
    const int j = threadIdx.x % half;        // pair index
    const int hg = threadIdx.x / half;       // head lane group
    const int ngroups = NT / half;
    const double theta = pow((double)base, -2.0 * (double)j / (double)dh);
    double sd, cd;
    sincos((double)pos * theta, &sd, &cd);
    const float sn = (float)sd, cs = (float)cd;
    const int nh = hq + 2 * hkv;
    const int ncols = nh * dh;
    const long cap = seqs.cap[s];
    for (int h = hg; h < nh; h += ngroups) {
        const float a = partial_sum(qkv, r, h * dh + j, ncols);
        const float b = partial_sum(qkv, r, h * dh + j + half, ncols);
        float ra = a, rb = b;
        if (h < hq + hkv) {
            ra = a * cs - b * sn;
            rb = a * sn + b * cs;
        }
        if (h < hq) {
            const long o = ((long)r * hq + h) * dh;
            if (F32) {
                ((float*)q_out)[o + j] = ra;
                ((float*)q_out)[o + j + half] = rb;
            } else {
                ((bf16_t*)q_out)[o + j] = f32_to_bf16(ra);
                ((bf16_t*)q_out)[o + j + half] = f32_to_bf16(rb);
            }
        } else {
            const int kind = h < hq + hkv ? 0 : 1;            // 0 = K, 1 = V
            const int kh = h - hq - kind * hkv;
            const long o = (((long)layer * 2 + kind) * hkv + kh) * cap * dh + (long)pos * dh;
            if (F32) {
                ((float*)seqs.kv[s])[o + j] = ra;
                ((float*)seqs.kv[s])[o + j + half] = rb;
            } else {
                ((bf16_t*)seqs.kv[s])[o + j] = f32_to_bf16(ra);
                ((bf16_t*)seqs.kv[s])[o + j + half] = f32_to_bf16(rb);
            }
        }
    }
}

void rope_kv(const Partials& qkv, int rows, const SeqTab& seqs, int layer, int n_layers, int hq, int hkv, int dh,
             float base, bool f32, void* q_out, hipStream_t st) {
    (void)n_layers;
    if (rows <= 0) return;
    if (f32)
        launch(rope_kv_kernel<true>, dim3(rows), dim3(NT), 0, st, qkv, seqs, layer, hq, hkv, dh, base, q_out);
    else
        launch(rope_kv_kernel<false>, dim3(rows), dim3(NT), 0, st, qkv, seqs, layer, hq, hkv, dh, base, q_out);
}

}  // namespace dlm
