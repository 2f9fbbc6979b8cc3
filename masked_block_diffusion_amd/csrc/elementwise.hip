// Row-wise kernels of the transformer block: embedding gather, RMSNorm with the
// GEMM-operand casts fused in (bf16, and per-token E4M3 for fp8 models),
// per-row E4M3 quantisation, and rotary embedding fused with the K/V cache
// write.  All are HBM/latency bound: one workgroup per token row, coalesced
// row accesses, deterministic fixed-order reductions.
#include "common.h"
#include "kernels.h"

namespace dlm {

constexpr int NT = 256;

__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x / WAVE;
    __syncthreads();
    if (threadIdx.x % WAVE == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) s += red[i];
    return s;
}

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
    hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(NT), 0, st, ids, table, dtype, d, vocab, mask_id,
                       (int)check_mask, x, err);
}

// ---------------------------------------------------------------- rmsnorm --

__global__ __launch_bounds__(NT) void rmsnorm_kernel(const float* x, const float* g, int d, float eps,
                                                      float* hf, bf16_t* hb, fp8_t* hq, float* hs) {
    __shared__ float red[NT / WAVE];
    const long r = blockIdx.x;
    const float* xr = x + r * d;
    float ss = 0.f;
    for (int c = threadIdx.x; c < d; c += NT) {
        const float v = xr[c];
        ss += v * v;
    }
    const float ms = block_sum(ss, red) / (float)d;
    const float den = sqrtf(ms + eps);
    float amax = 0.f;
    for (int c = threadIdx.x; c < d; c += NT) {
        const float h = xr[c] / den * g[c];
        if (hf) hf[r * d + c] = h;
        if (hb) {
            const bf16_t b = f32_to_bf16(h);
            hb[r * d + c] = b;
            amax = fmaxf(amax, fabsf(bf16_to_f32(b)));
        }
    }
    if (!hq) return;
    amax = block_max(amax, red);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    for (int c = threadIdx.x; c < d; c += NT) hq[r * d + c] = f32_to_e4m3(bf16_to_f32(hb[r * d + c]) / s);
    if (threadIdx.x == 0) hs[r] = s;
}

void rmsnorm(const float* x, const float* g, int rows, int d, float eps, float* hf, uint16_t* hb,
             uint8_t* hq, float* hs, hipStream_t st) {
    if (rows <= 0) return;
    hipLaunchKernelGGL(rmsnorm_kernel, dim3(rows), dim3(NT), 0, st, x, g, d, eps, hf, hb, hq, hs);
}

// ------------------------------------------------------------- quant_rows --

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
    hipLaunchKernelGGL(quant_rows_kernel, dim3(rows), dim3(NT), 0, st, x, d, q, s);
}

// ---------------------------------------------------------------- rope_kv --
// Rotate-half rotary embedding: for i < dh/2 the pair (v[i], v[i + dh/2]) is
// rotated by pos * base^(-2i/dh).  The angle and its sine/cosine are formed in
// double precision (positions reach several thousand), then applied in fp32.

template <bool F32>
__global__ __launch_bounds__(NT) void rope_kv_kernel(const float* qkv, SeqTab seqs, int layer, int hq,
                                                      int hkv, int dh, float base, void* q_out) {
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
    const float* row = qkv + (long)r * nh * dh;
    const long cap = seqs.cap[s];
    for (int h = hg; h < nh; h += ngroups) {
        const float a = row[h * dh + j], b = row[h * dh + j + half];
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

void rope_kv(const float* qkv, int rows, const SeqTab& seqs, int layer, int n_layers, int hq, int hkv,
             int dh, float base, bool f32, void* q_out, hipStream_t st) {
    (void)n_layers;
    if (rows <= 0) return;
    if (f32)
        hipLaunchKernelGGL(rope_kv_kernel<true>, dim3(rows), dim3(NT), 0, st, qkv, seqs, layer, hq, hkv, dh,
                           base, q_out);
    else
        hipLaunchKernelGGL(rope_kv_kernel<false>, dim3(rows), dim3(NT), 0, st, qkv, seqs, layer, hq, hkv, dh,
                           base, q_out);
}

}  // namespace dlm
