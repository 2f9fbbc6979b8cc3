// Prediction and commit for gfx950.
//
//  lm_merge  per canvas row, folds the LM-head GEMM's per-vocab-tile partials
//            (tile max, lowest argmax, sum exp(l - tile max)) into the row's
//            prediction (lowest-id argmax over the vocabulary without [MASK])
//            and confidence = max softmax probability = 1 / sum exp(l - max).
//            One wave per row; fixed lane/tile assignment, so deterministic.
//  commit    one workgroup per request.  Each masked position's rank is the
//            number of masked positions that beat it (higher confidence, or
//            equal confidence and a lower position) -- an exact, total order.
//            Top-k rule: commit rank < k.  Threshold rule: commit conf >= thr
//            or rank 0 (if any masked position reaches thr, the rank-0 one
//            does, so "at least the most confident one" is exactly this).
//            Forced fill: commit every masked position.  Only [MASK] entries
//            are written, always with the prediction.
#include "common.h"
#include "kernels.h"

namespace dlm {

constexpr int LM_UNROLL = 8;

__global__ __launch_bounds__(256) void lm_merge_kernel(const float* pmax, const float* psum, const int* pidx,
                                                        int rows, int n_tiles, float* conf, int* pred) {
    const int lane = threadIdx.x % WAVE;
    const int r = blockIdx.x * 4 + threadIdx.x / WAVE;
    if (r >= rows) return;
    const float* pm = pmax + (long)r * n_tiles;
    const float* ps = psum + (long)r * n_tiles;
    const int* pi = pidx + (long)r * n_tiles;
    // a lane takes tiles lane, lane + 64, ...; each pass loads LM_UNROLL of
    // them before using any (one dependent round trip per tile otherwise)
    float m = -INFINITY;
    int ix = 0x7fffffff;
    for (int t0 = lane; t0 < n_tiles; t0 += WAVE * LM_UNROLL) {
        float v[LM_UNROLL];
        int id[LM_UNROLL];
#pragma unroll
        for (int u = 0; u < LM_UNROLL; ++u) {
            const int t = t0 + u * WAVE;
            v[u] = t < n_tiles ? pm[t] : -INFINITY;
            id[u] = t < n_tiles ? pi[t] : 0x7fffffff;
        }
#pragma unroll
        for (int u = 0; u < LM_UNROLL; ++u)
            if (v[u] > m || (v[u] == m && id[u] < ix)) { m = v[u]; ix = id[u]; }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(m, o, WAVE);
        const int oi = __shfl_xor(ix, o, WAVE);
        if (om > m || (om == m && oi < ix)) { m = om; ix = oi; }
    }
    float z = 0.f;
    for (int t0 = lane; t0 < n_tiles; t0 += WAVE * LM_UNROLL) {
        float v[LM_UNROLL], w[LM_UNROLL];
#pragma unroll
        for (int u = 0; u < LM_UNROLL; ++u) {
            const int t = t0 + u * WAVE;
            v[u] = t < n_tiles ? pm[t] : -INFINITY;
            w[u] = t < n_tiles ? ps[t] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < LM_UNROLL; ++u)
            if (v[u] != -INFINITY) z += w[u] * __expf(v[u] - m);
    }
    z = wave_sum(z);
    if (lane == 0) {
        conf[r] = 1.0f / z;
        pred[r] = ix;
    }
}

void lm_merge(const float* pmax, const float* psum, const int* pidx, int rows, int n_tiles, float* conf, int* pred,
              hipStream_t st) {
    if (rows <= 0) return;
    launch(lm_merge_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, pmax, psum, pidx, rows, n_tiles,
                       conf, pred);
}

struct CanvasTab {
    int32_t* c[MAX_SEQS];
};

constexpr int CMAX = 1024;

// Ranking keys: a masked position's confidence, -inf for the others.  A
// confidence is 1 / (sum of exp terms, the largest being 1), in (0, 1], so a
// -inf key never beats or ties a masked one: counting the keys that beat a
// masked position over all positions counts exactly the masked ones.  The
// keys are read four at a time (independent loads, not one dependent chain).
__global__ __launch_bounds__(256) void commit_kernel(CanvasTab tab, int C, const float* conf, const int* pred,
                                                      int mask_id, int kind, int k, float thr, int force_all,
                                                      float edit_thr, int* n_committed, int* n_masked) {
    __shared__ __attribute__((aligned(16))) float key[CMAX];
    __shared__ int cnt[2];
    const int s = blockIdx.x;
    int32_t* canvas = tab.c[s];
    const float* cf = conf + (long)s * C;
    const int* pr = pred + (long)s * C;
    const int C4 = (C + 3) / 4;
    if (threadIdx.x < 2) cnt[threadIdx.x] = 0;
    for (int j = threadIdx.x; j < 4 * C4; j += 256) key[j] = (j < C && canvas[j] == mask_id) ? cf[j] : -INFINITY;
    __syncthreads();
    int my_commit = 0, my_left = 0;
    for (int j = threadIdx.x; j < C; j += 256) {
        const float cj = key[j];
        if (cj == -INFINITY) {
            // token editing: an earlier token whose prediction moved with enough confidence
            if (edit_thr > 0.f && pr[j] != canvas[j] && cf[j] >= edit_thr) {
                canvas[j] = pr[j];
                ++my_commit;
            }
            continue;
        }
        // rank = #{i < j: key_i >= cj} + #{i > j: key_i > cj}
        int rank = 0;
        const f32x4* k4 = (const f32x4*)key;
#pragma unroll 8
        for (int q = 0; q < C4; ++q) {
            const f32x4 v = k4[q];
            const int i = 4 * q;
            rank += (i + 0 < j) ? (v[0] >= cj) : (v[0] > cj);
            rank += (i + 1 < j) ? (v[1] >= cj) : (v[1] > cj);
            rank += (i + 2 < j) ? (v[2] >= cj) : (v[2] > cj);
            rank += (i + 3 < j) ? (v[3] >= cj) : (v[3] > cj);
        }
        bool take;
        if (force_all) take = true;
        else if (kind == 0) take = rank < k;
        else take = (cj >= thr) || rank == 0;
        if (take) {
            canvas[j] = pr[j];
            ++my_commit;
        } else {
            ++my_left;
        }
    }
    atomicAdd(&cnt[0], my_commit);
    atomicAdd(&cnt[1], my_left);
    __syncthreads();
    if (threadIdx.x == 0) {
        if (n_committed) n_committed[s] = cnt[0];
        if (n_masked) n_masked[s] = cnt[1];
    }
}

void commit(int32_t* const* canvases, int n_seqs, int C, const float* conf, const int* pred, int mask_id, int kind,
            int k, float thr, bool force_all, float edit_thr, int* n_committed, int* n_masked, hipStream_t st) {
    if (n_seqs <= 0) return;
    CanvasTab tab;
    for (int i = 0; i < n_seqs; ++i) tab.c[i] = canvases[i];
    launch(commit_kernel, dim3(n_seqs), dim3(256), 0, st, tab, C, conf, pred, mask_id, kind, k, thr,
                       (int)force_all, edit_thr, n_committed, n_masked);
}

}  // namespace dlm
