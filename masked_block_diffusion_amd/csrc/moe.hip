// Mixture-of-experts routing for gfx950.
//
//  router_topk  one wave per token row: the router logits (the router GEMM's
//               split-K partials summed here, in split order), the top-k
//               experts by logit (ties -> lower expert id; the same order as
//               by probability) found by ranking every logit against the row,
//               and their softmax probabilities renormalised over the chosen k
//               (the full softmax denominator cancels).
//  moe_route    stable counting sort of the rows * k assignments by expert, so
//               each expert's rows are contiguous for the grouped GEMM.  Up to
//               ROUTE_FUSED_MAX assignments (a canvas step): one workgroup
//               does it all -- one assignment per lane, its rank among the
//               lanes of its wave with the same expert from ballots, counts per
//               (64-assignment chunk, expert), bases by scans.  Beyond
//               that (prefill, large batches), three kernels:
//                 hist     per 256-assignment block: per-expert counts and each
//                          assignment's rank among earlier same-expert ones;
//                 scan     per-expert totals -> offsets, per-block bases, and the
//                          first m-tile of every expert (bm-row tiles);
//                 scatter  sorted position of every assignment and its inverse.
//               Integer-only and deterministic: order is (expert, row, slot).
// The weighted un-permute of the experts' outputs (x += sum over slots of
// w * y) is done by the RMSNorm that reads x next (MoeGather).
#include "common.h"
#include "kernels.h"

namespace dlm {

constexpr int MAX_E = 256;

// One wave per row, four rows per workgroup.  The row's logits are staged in
// LDS; logit e's rank is the number of logits that beat it (larger, or equal
// with a lower expert id), so the experts of rank < k in rank order are the
// top-k in selection order.  Their probabilities exp(l - max) go to slot
// `rank` and are summed in slot order for the renormalisation.
__global__ __launch_bounds__(256) void router_topk_kernel(Partials logits, int rows, int E, int k, int* ids,
                                                           float* w, int* ids_copy, float* logits_copy) {
    __shared__ __attribute__((aligned(16))) float sv[4][MAX_E];
    __shared__ float sp[4][16];
    const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
    const int r = blockIdx.x * 4 + wv;
    const bool live = r < rows;                      // every wave reaches both barriers
    constexpr int PER = MAX_E / WAVE;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + WAVE * j;
        v[j] = -INFINITY;
        if (live && e < E) {
            float x = 0.f;
            for (int s = 0; s < logits.splits; ++s) x += logits.p[s * logits.stride + (long)r * E + e];
            v[j] = x;
            if (logits_copy) logits_copy[(long)r * E + e] = x;
        }
        sv[wv][e] = v[j];
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < PER; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    __syncthreads();
    const int E4 = (E + 3) / 4;
    const f32x4* k4 = (const f32x4*)sv[wv];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int e = lane + WAVE * j;
        if (!live || e >= E) continue;
        const float c = v[j];
        int rank = 0;
        for (int q = 0; q < E4; ++q) {
            const f32x4 x = k4[q];
            const int i = 4 * q;
            rank += (i + 0 < e) ? (x[0] >= c) : (x[0] > c);
            rank += (i + 1 < e) ? (x[1] >= c) : (x[1] > c);
            rank += (i + 2 < e) ? (x[2] >= c) : (x[2] > c);
            rank += (i + 3 < e) ? (x[3] >= c) : (x[3] > c);
        }
        if (rank < k) {
            sp[wv][rank] = expf(c - m);
            ids[(long)r * k + rank] = e;
            if (ids_copy) ids_copy[(long)r * k + rank] = e;
        }
    }
    __syncthreads();
    if (live && lane < k) {
        float sel_sum = 0.f;
        for (int s = 0; s < k; ++s) sel_sum += sp[wv][s];
        w[(long)r * k + lane] = sp[wv][lane] / sel_sum;
    }
}

void router_topk(const Partials& logits, int rows, int E, int k, int* ids, float* w, int* ids_copy,
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

// One workgroup of 256 threads: thread e owns expert e.  An expert's block
// counts lie E ints apart; each pass over them issues SCAN_CHUNK loads before
// using any (a chain of one dependent load per block took 86-92 us for the
// 128-256 blocks of a 4096-token prompt or a 32-request step).  Pass 1 sums them, then the expert totals and m-tile counts are
// scanned, pass 2 writes each block's base: the expert's offset plus the
// counts of the earlier blocks.
constexpr int SCAN_CHUNK = 32;

__global__ __launch_bounds__(256) void route_scan_kernel(int* hist, int nblocks, int E, int bm, int* offs,
                                                          int* tile_start) {
    __shared__ int tot[MAX_E], tiles[MAX_E];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int b0 = 0; b0 < nblocks; b0 += SCAN_CHUNK) {
            int c[SCAN_CHUNK];
#pragma unroll
            for (int i = 0; i < SCAN_CHUNK; ++i) c[i] = b0 + i < nblocks ? hist[(long)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < SCAN_CHUNK; ++i) run += c[i];
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
        int base = tot[e];
        for (int b0 = 0; b0 < nblocks; b0 += SCAN_CHUNK) {
            int c[SCAN_CHUNK];
#pragma unroll
            for (int i = 0; i < SCAN_CHUNK; ++i) c[i] = b0 + i < nblocks ? hist[(long)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < SCAN_CHUNK; ++i) {
                if (b0 + i < nblocks) hist[(long)(b0 + i) * E + e] = base;   // base of block b0 + i within the sort
                base += c[i];
            }
        }
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

constexpr int RF_THREADS = 1024;
constexpr int RF_WAVES = RF_THREADS / WAVE;
constexpr int ROUTE_FUSED_MAX = 4096;
constexpr int RF_CHUNKS = ROUTE_FUSED_MAX / WAVE;   // 64-assignment chunks
constexpr int RF_PER_WAVE = RF_CHUNKS / RF_WAVES;   // chunks per wave

// Chunk c (assignments 64c .. 64c + 63) goes to wave c % RF_WAVES, one
// assignment per lane.  Lanes holding the same expert are found with one
// ballot per bit of the expert id; a lane's rank among them is the popcount of
// the lower ones, and the lowest records the chunk's count in cnt[c][e].
// Then per expert an exclusive prefix over chunks, an exclusive scan over
// experts (one wave, shuffles), and position = offs[e] + cnt[c][e] + rank:
// the (expert, assignment) order.
__global__ __launch_bounds__(RF_THREADS) void route_fused_kernel(const int* ids, int n_assign, int E, int bm,
                                                                 int* offs, int* tile_start, int* sorted_assign,
                                                                 int* inv) {
    __shared__ int cnt[RF_CHUNKS * MAX_E];           // [chunk][expert]: counts, then bases within the expert
    __shared__ int tot[MAX_E + 1], tiles[MAX_E + 1];
    const int t = threadIdx.x, lane = t % WAVE, w = t / WAVE;
    const int nchunks = (n_assign + WAVE - 1) / WAVE;
    for (int i = t; i < nchunks * E; i += RF_THREADS) cnt[i] = 0;
    __syncthreads();
    int ex[RF_PER_WAVE], rank[RF_PER_WAVE];
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < RF_PER_WAVE; ++j) {
        const int c = w + j * RF_WAVES;
        const int a = c * WAVE + lane;
        const bool valid = c < nchunks && a < n_assign;
        const int e = valid ? ids[a] : 0;
        unsigned long long m = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {            // E <= 256
            const bool bit = (e >> b) & 1;
            const unsigned long long bb = __ballot(bit);
            m &= bit ? bb : ~bb;
        }
        ex[j] = e;
        rank[j] = __popcll(m & below);
        if (valid && rank[j] == 0) cnt[c * E + e] = __popcll(m);
    }
    __syncthreads();
    if (t < E) {
        int run = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int v = cnt[c * E + t];
            cnt[c * E + t] = run;
            run += v;
        }
        tot[t] = run;
    }
    __syncthreads();
    if (w == 0) {
        // exclusive scans of the totals and of their m-tile counts; lane l
        // holds experts 4l .. 4l + 3
        int n[4], tl[4], sn = 0, st = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            n[i] = e < E ? tot[e] : 0;
            tl[i] = (n[i] + bm - 1) / bm;
            sn += n[i];
            st += tl[i];
        }
        int in = sn, it = st;                      // inclusive scan over lanes
#pragma unroll
        for (int o = 1; o < WAVE; o <<= 1) {
            const int pn = __shfl_up(in, o, WAVE), pt = __shfl_up(it, o, WAVE);
            if (lane >= o) { in += pn; it += pt; }
        }
        int on = in - sn, ot = it - st;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = 4 * lane + i;
            if (e < E) { tot[e] = on; tiles[e] = ot; }
            on += n[i];
            ot += tl[i];
        }
        if (lane == WAVE - 1) { tot[E] = in; tiles[E] = it; }   // the grand totals
    }
    __syncthreads();
    if (t <= E) {
        offs[t] = tot[t];
        tile_start[t] = tiles[t];
    }
#pragma unroll
    for (int j = 0; j < RF_PER_WAVE; ++j) {
        const int c = w + j * RF_WAVES;
        const int a = c * WAVE + lane;
        if (c < nchunks && a < n_assign) {
            const int pos = tot[ex[j]] + cnt[c * E + ex[j]] + rank[j];
            sorted_assign[pos] = a;
            inv[a] = pos;
        }
    }
}

void moe_route(const int* ids, int n_assign, int E, int bm, int* offs, int* tile_start, int* sorted_assign, int* inv,
               const RouteWork& w, hipStream_t st) {
    const int nb = route_blocks(n_assign);
    if (nb == 0) return;
    if (n_assign <= ROUTE_FUSED_MAX && E <= MAX_E) {
        launch(route_fused_kernel, dim3(1), dim3(RF_THREADS), 0, st, ids, n_assign, E, bm, offs, tile_start,
               sorted_assign, inv);
        return;
    }
    launch(route_hist_kernel, dim3(nb), dim3(RB), 0, st, ids, n_assign, E, w.hist, w.local_rank);
    launch(route_scan_kernel, dim3(1), dim3(256), 0, st, w.hist, nb, E, bm, offs, tile_start);
    launch(route_scatter_kernel, dim3(nb), dim3(RB), 0, st, ids, n_assign, E, w.hist, w.local_rank,
                       sorted_assign, inv);
}

}  // namespace dlm
