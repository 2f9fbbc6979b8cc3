// Mixture-of-experts routing for gfx950.
//
//  router_topk  one wave per token row: softmax over the E router logits, the
//               top-k experts by logit (ties -> lower expert id; the same order
//               as by probability), and their probabilities renormalised over
//               the chosen k (the full softmax denominator cancels).
//  moe_route    stable counting sort of the rows * k assignments by expert, so
//               each expert's rows are contiguous for the grouped GEMM:
//                 hist     per 256-assignment block: per-expert counts and each
//                          assignment's rank among earlier same-expert ones;
//                 scan     per-expert totals -> offsets, per-block bases, and the
//                          first m-tile of every expert (GROUPED_BM-row tiles);
//                 scatter  sorted position of every assignment and its inverse.
//               Integer-only and deterministic: order is (expert, row, slot).
//  moe_combine  x[r] += sum over slots s (in selection order) of
//               w[r, s] * y[inv[r * k + s]].
#include "common.h"
#include "kernels.h"

namespace dlm {

constexpr int MAX_E = 256;

__global__ __launch_bounds__(256) void router_topk_kernel(const float* logits, int rows, int E, int k, int* ids,
                                                           float* w, int* ids_copy, float* logits_copy) {
    const int lane = threadIdx.x % WAVE;
    const int r = blockIdx.x * 4 + threadIdx.x / WAVE;
    if (r >= rows) return;
    constexpr int PER = MAX_E / WAVE;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + WAVE * j;
        v[j] = e < E ? logits[(long)r * E + e] : -INFINITY;
        if (logits_copy && e < E) logits_copy[(long)r * E + e] = v[j];
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < PER; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    float sel_sum = 0.f;
    for (int s = 0; s < k; ++s) {
        // best remaining (value, lowest id) in this lane, then across the wave
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int e = lane + WAVE * j;
            if (e < E && (v[j] > bv || (v[j] == bv && e < be))) { bv = v[j]; be = e; }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o, WAVE);
            const int oe = __shfl_xor(be, o, WAVE);
            if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
        }
        const float p = expf(bv - m);
        sel_sum += p;
        if (lane == 0) {
            ids[(long)r * k + s] = be;
            if (ids_copy) ids_copy[(long)r * k + s] = be;
            w[(long)r * k + s] = p;
        }
        // retire the chosen expert (k <= E, so a remaining one always exists)
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (lane + WAVE * j == be) v[j] = -INFINITY;
    }
    if (lane == 0)
        for (int s = 0; s < k; ++s) w[(long)r * k + s] /= sel_sum;
}

void router_topk(const float* logits, int rows, int E, int k, int* ids, float* w, int* ids_copy,
                 float* logits_copy, hipStream_t st) {
    if (rows <= 0) return;
    launch(router_topk_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, logits, rows, E, k, ids, w,
                       ids_copy, logits_copy);
}

// ------------------------------------------------------------------ route --

constexpr int RB = 256;   // assignments per block

int route_blocks(int n_assign) { return (n_assign + RB - 1) / RB; }

__global__ __launch_bounds__(RB) void route_hist_kernel(const int* ids, int n_assign, int E, int* hist,
                                                         int* local_rank) {
    __shared__ int sid[RB];
    const int b = blockIdx.x, t = threadIdx.x;
    const int a = b * RB + t;
    sid[t] = a < n_assign ? ids[a] : -1;
    __syncthreads();
    if (a < n_assign) {
        const int e = sid[t];
        int rank = 0;
        for (int i = 0; i < t; ++i) rank += (sid[i] == e);
        local_rank[a] = rank;
    }
    if (t < E) {
        int c = 0;
        for (int i = 0; i < RB; ++i) c += (sid[i] == t);
        hist[(long)b * E + t] = c;
    }
}

// One workgroup of 256 threads: thread e owns expert e.
__global__ __launch_bounds__(256) void route_scan_kernel(int* hist, int nblocks, int E, int bm, int* offs,
                                                          int* tile_start) {
    __shared__ int tot[MAX_E], tiles[MAX_E];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int b = 0; b < nblocks; ++b) {
            const int c = hist[(long)b * E + e];
            hist[(long)b * E + e] = run;       // base of block b within expert e
            run += c;
        }
    }
    tot[e] = e < E ? run : 0;
    tiles[e] = e < E ? (run + bm - 1) / bm : 0;
    __syncthreads();
    if (e == 0) {
        int o = 0, t = 0;
        for (int i = 0; i < E; ++i) {
            const int c = tot[i], n = tiles[i];
            tot[i] = o;
            tiles[i] = t;
            o += c;
            t += n;
        }
        offs[E] = o;
        tile_start[E] = t;
    }
    __syncthreads();
    if (e < E) {
        offs[e] = tot[e];
        tile_start[e] = tiles[e];
        for (int b = 0; b < nblocks; ++b) hist[(long)b * E + e] += tot[e];
    }
}

__global__ __launch_bounds__(RB) void route_scatter_kernel(const int* ids, int n_assign, int E, const int* hist,
                                                            const int* local_rank, int* sorted_assign, int* inv) {
    const int a = blockIdx.x * RB + threadIdx.x;
    if (a >= n_assign) return;
    const int p = hist[(long)blockIdx.x * E + ids[a]] + local_rank[a];
    sorted_assign[p] = a;
    inv[a] = p;
}

void moe_route(const int* ids, int n_assign, int E, int* offs, int* tile_start, int* sorted_assign, int* inv,
               const RouteWork& w, hipStream_t st) {
    const int nb = route_blocks(n_assign);
    if (nb == 0) return;
    launch(route_hist_kernel, dim3(nb), dim3(RB), 0, st, ids, n_assign, E, w.hist, w.local_rank);
    launch(route_scan_kernel, dim3(1), dim3(256), 0, st, w.hist, nb, E, GROUPED_BM, offs, tile_start);
    launch(route_scatter_kernel, dim3(nb), dim3(RB), 0, st, ids, n_assign, E, w.hist, w.local_rank,
                       sorted_assign, inv);
}

// ---------------------------------------------------------------- combine --

// One workgroup per (token row, 1024-column chunk); each thread owns 4
// consecutive columns (d is a multiple of 4) and issues all of its loads
// before the arithmetic: x += shared-expert output (split partials summed in
// order, fp8 scales applied) + sum over the row's k slots of w * y[slot's
// sorted row].
constexpr int COMBINE_COLS = 1024;
__global__ __launch_bounds__(256) void moe_combine_kernel(float* x, Partials shared, const float* y,
                                                           const int* inv, const float* w, int k, int d) {
    const long r = blockIdx.x;
    const int c = blockIdx.y * COMBINE_COLS + 4 * threadIdx.x;
    if (c >= d) return;
    const float* wr = w + r * k;
    const int* ir = inv + r * k;
    f32x4 yv[16];
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < k) yv[s] = *(const f32x4*)(y + (long)ir[s] * d + c);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (shared.p) {
        const long off = r * d + c;
        for (int s = 0; s < shared.splits; ++s) acc += *(const f32x4*)(shared.p + s * shared.stride + off);
        if (shared.a_scale) acc = acc * shared.a_scale[r] * *(const f32x4*)(shared.b_scale + c);
    }
    f32x4* xp = (f32x4*)(x + r * d + c);
    const f32x4 x0 = *xp;
#pragma unroll
    for (int s = 0; s < 16; ++s)
        if (s < k) acc += wr[s] * yv[s];
    *xp = x0 + acc;
}

void moe_combine(float* x, const Partials& shared, const float* y, const int* inv, const float* w, int rows, int k,
                 int d, hipStream_t st) {
    if (rows <= 0) return;
    launch(moe_combine_kernel, dim3(rows, (d + COMBINE_COLS - 1) / COMBINE_COLS), dim3(256), 0, st, x, shared, y, inv, w, k,
           d);
}

}  // namespace dlm
