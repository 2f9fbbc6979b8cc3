// C ABI of the block-diffusion denoising library: argument validation,
// workspace planning, and the sequence of gfx950 kernels that makes up prefill,
// one denoising step, the commit, and the canvas append.  The operations and
// their sources are documented in include/dlm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dlm.h"
#include "kernels.h"

using namespace dlm;

namespace dlm {
LaunchTimer*& launch_timer() {
    thread_local LaunchTimer* t = nullptr;
    return t;
}
}  // namespace dlm

// Workspace of dlm_denoise_step_noalloc: one copy per device, allocated when
// the library's code object is loaded there.  Host code never uses this name
// as an address (on the host it is only a handle): dlm_create looks up the
// device address once per device with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[DLM_STATIC_SCRATCH_BYTES];

namespace {

thread_local std::string g_err;

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

// Device address of `scratch` on the current device `dev` (looked up once).
hipError_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

dlm_status fail(dlm_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dlm_status fail(dlm_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

const char* kKernelNames[DLM_K_COUNT] = {
    "embed", "rmsnorm", "gemm_qkv", "rope_kv", "attention", "attention_merge", "gemm_o",
    "gemm_gate_up", "gemm_down", "quant", "router", "router_topk", "moe_route", "expert_gate_up",
    "expert_down", "moe_combine", "lm_head", "lm_merge", "commit", "splitk_epilogue"};

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_bytes(int dtype) { return dtype == DLM_F32 ? 4 : dtype == DLM_BF16 ? 2 : 1; }

}  // namespace

struct dlm_model {
    dlm_config cfg;
    dlm_weights w;
    std::vector<dlm_layer_weights> layers;
    int* d_err = nullptr;
    int device = 0;
    void* scratch = nullptr;         // this device's static workspace (dlm_denoise_step_noalloc)
    // MoE models: the shared expert runs on a second stream of the library's
    // own (default priority), forked from and joined back into the caller's
    // stream with these events, so it overlaps the routing chain
    hipStream_t side = nullptr;
    hipEvent_t fork_ev = nullptr, join_ev = nullptr;
    int32_t* dbg_router = nullptr;   // test hook: per-layer router choices
    float* dbg_router_logits = nullptr;
    int64_t dbg_cap = 0;             // (layer, row) pairs the hook buffers hold
    // timing
    uint32_t timing_mask = 0;
    struct Ev { hipEvent_t a, b; int id; };
    std::vector<Ev> pending;
    std::vector<hipEvent_t> pool;
    float ms[DLM_K_COUNT] = {};
    int launches[DLM_K_COUNT] = {};
};

namespace {

// RAII scope around one kernel launch of a timed kernel id: the first kernel
// launched in the scope carries the start / stop events in its dispatch.
// With install = false the timer is only prepared (timer() hands it to a
// launcher that arms it for a specific kernel of its own).
struct Timed {
    dlm_model* m; int id; bool on, installed = false;
    LaunchTimer lt;
    LaunchTimer* prev = nullptr;
    Timed(dlm_model* m_, int id_, hipStream_t, bool install = true) : m(m_), id(id_) {
        on = (m->timing_mask >> id) & 1u;
        if (!on) return;
        lt.start = take();
        lt.stop = take();
        lt.armed = true;
        if (install) {
            installed = true;
            prev = launch_timer();
            launch_timer() = &lt;
        }
    }
    LaunchTimer* timer() { return on ? &lt : nullptr; }
    ~Timed() {
        if (!on) return;
        if (installed) launch_timer() = prev;
        if (lt.armed) {                  // nothing launched (empty problem)
            m->pool.push_back(lt.start);
            m->pool.push_back(lt.stop);
        } else {
            m->pending.push_back({lt.start, lt.stop, id});
        }
    }
    hipEvent_t take() {
        if (!m->pool.empty()) {
            hipEvent_t e = m->pool.back();
            m->pool.pop_back();
            return e;
        }
        hipEvent_t e;
        hipEventCreate(&e);
        return e;
    }
};

// ----------------------------------------------------------- workspace --

struct Plan {
    size_t x, hA, hb, hq, hs, qkv, q, ao, aoq, aos, fi, fiq, fis, rl, tid, tw, offs, tstart, sorted, inv,
        hist, lrank, ei, eiq, eis, y, pmax, psum, pidx, opart, mlpart, splitk, splitk2, total;
    long splitk_floats;
};

// Largest split-K partial space any dense GEMM of a forward over `rows` rows uses.
long splitk_need(const dlm_config& c, int rows) {
    const int d = c.d_model, qd = c.n_q_heads * c.head_dim;
    const int nqkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
    auto need = [&](int dtype, int epi, int N, int K) {
        GemmDesc g;
        g.dtype = dtype; g.epi = epi; g.out_f32 = c.dtype == DLM_F32;
        g.M = rows; g.N = N; g.K = K;
        return gemm_splitk_floats(g);
    };
    long m = 0;
    m = std::max(m, need(c.dtype, GEMM_STORE_F32, nqkv, d));
    m = std::max(m, need(c.dtype, GEMM_ADD_F32, d, qd));
    m = std::max(m, need(c.dtype, GEMM_SWIGLU, c.d_ffn, d));
    m = std::max(m, need(c.dtype, GEMM_ADD_F32, d, c.d_ffn));
    if (c.ffn == DLM_FFN_MOE)
        m = std::max(m, need(c.dtype == DLM_F32 ? DT_F32 : DT_BF16, GEMM_STORE_F32, c.n_experts, d));
    return m;
}

Plan plan(const dlm_config& c, int rows, int max_kv) {
    (void)max_kv;
    Plan p{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off += align_up(bytes);
        return o;
    };
    const size_t R = rows, d = c.d_model, qd = (size_t)c.n_q_heads * c.head_dim;
    const size_t nqkv = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
    const size_t act = c.dtype == DLM_F32 ? 4 : 2;
    const bool fp8 = c.dtype == DLM_FP8;
    const bool moe = c.ffn == DLM_FFN_MOE;
    const size_t A = moe ? R * c.top_k : 0;
    p.x = take(R * d * 4);
    p.hA = take(R * d * act);                // fp32 (f32) or bf16 normalised activations
    p.hb = p.hA;
    p.hq = fp8 ? take(R * d) : 0;
    p.hs = fp8 ? take(R * 4) : 0;
    p.qkv = take(R * nqkv * 4);
    p.q = take(R * qd * act);
    p.ao = take(R * qd * act);
    p.aoq = fp8 ? take(R * qd) : 0;
    p.aos = fp8 ? take(R * 4) : 0;
    p.fi = take(R * c.d_ffn * act);
    p.fiq = fp8 ? take(R * c.d_ffn) : 0;
    p.fis = fp8 ? take(R * 4) : 0;
    if (moe) {
        p.rl = take(R * c.n_experts * 4);
        p.tid = take(A * 4);
        p.tw = take(A * 4);
        p.offs = take((c.n_experts + 1) * 4);
        p.tstart = take((c.n_experts + 1) * 4);
        p.sorted = take(A * 4);
        p.inv = take(A * 4);
        p.hist = take((size_t)route_blocks((int)A) * c.n_experts * 4);
        p.lrank = take(A * 4);
        p.ei = take(A * c.d_expert * act);
        p.eiq = fp8 ? take(A * c.d_expert) : 0;
        p.eis = fp8 ? take(A * 4) : 0;
        p.y = take(A * d * 4);
    }
    const int tn = std::min(lm_head_tile_n(1), lm_head_tile_n(1 << 20));         // the narrowest vocab slice
    const size_t nt = (c.vocab + tn - 1) / tn;
    p.pmax = take(R * nt * 4);
    p.psum = take(R * nt * 4);
    p.pidx = take(R * nt * 4);
    const size_t af = attention_work_floats(rows, c.n_q_heads, c.head_dim);
    p.opart = take(af / (c.head_dim + 2) * c.head_dim * 4);
    p.mlpart = take(af / (c.head_dim + 2) * 2 * 4);
    p.splitk_floats = splitk_need(c, rows);
    p.splitk = take(std::max(1L, p.splitk_floats) * 4);
    p.splitk2 = moe ? take(std::max(1L, p.splitk_floats) * 4) : p.splitk;   // the shared expert's own
    p.total = off;
    return p;
}

template <typename T> T* at(void* ws, size_t off) { return (T*)((uint8_t*)ws + off); }

// ------------------------------------------------------------- validation --

dlm_status check_config(const dlm_config* c) {
    if (!c) return fail(DLM_E_ARG, "config is NULL");
    if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->vocab < 2)
        return fail(DLM_E_SHAPE, "non-positive model dimension");
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
        return fail(DLM_E_SHAPE, "head_dim %d not in {32, 64, 128}", c->head_dim);
    if (c->n_q_heads % c->n_kv_heads) return fail(DLM_E_SHAPE, "n_q_heads %% n_kv_heads != 0");
    if (c->head_dim >= 32 && (c->n_q_heads + c->n_kv_heads) * c->head_dim > 8192)
        return fail(DLM_E_SHAPE, "(n_q_heads + n_kv_heads) * head_dim %d exceeds 8192",
                    (c->n_q_heads + c->n_kv_heads) * c->head_dim);
    if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(DLM_E_ARG, "mask_id outside [0, vocab)");
    if (c->dtype < DLM_F32 || c->dtype > DLM_FP8) return fail(DLM_E_DTYPE, "unknown dtype %d", c->dtype);
    if (c->ffn != DLM_FFN_DENSE && c->ffn != DLM_FFN_MOE) return fail(DLM_E_ARG, "unknown ffn kind %d", c->ffn);
    if (c->canvas < 1 || c->canvas > 1024) return fail(DLM_E_SHAPE, "canvas %d not in [1, 1024]", c->canvas);
    if (c->d_ffn < 1) return fail(DLM_E_SHAPE, "d_ffn < 1");
    if (c->d_model > rmsnorm_max_dim()) return fail(DLM_E_SHAPE, "d_model above %d", rmsnorm_max_dim());
    if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f)) return fail(DLM_E_ARG, "bad rms_eps / rope_base");
    const int eb = elem_bytes(c->dtype);
    const int kdims[4] = {c->d_model, c->n_q_heads * c->head_dim, c->d_ffn,
                          c->ffn == DLM_FFN_MOE ? c->d_expert : c->d_model};
    for (int k : kdims)
        if ((k * eb) % 128) return fail(DLM_E_SHAPE, "GEMM inner dimension %d is not a multiple of 128 bytes", k);
    if (c->ffn == DLM_FFN_MOE) {
        if (c->n_experts < 1 || c->n_experts > 256) return fail(DLM_E_SHAPE, "n_experts not in [1, 256]");
        if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts)
            return fail(DLM_E_SHAPE, "top_k not in [1, min(16, n_experts)]");
        if (c->d_expert < 1) return fail(DLM_E_SHAPE, "d_expert < 1");
        if (c->expert_dtype != c->dtype) {
            if ((c->expert_dtype != DLM_MXFP4 && c->expert_dtype != DLM_MXFP6) || c->dtype != DLM_BF16)
                return fail(DLM_E_DTYPE, "expert_dtype %d with dtype %d (experts: the model's dtype, or MXFP4 / "
                            "MXFP6 with bf16)", c->expert_dtype, c->dtype);
            if (c->d_model % 128 || c->d_expert % 128)
                return fail(DLM_E_SHAPE, "MX experts need d_model and d_expert multiples of 128");
        }
    }
    return DLM_OK;
}

// Element bits of the routed experts' MX weights, 0 when they are not MX.
int mx_bits(const dlm_config& c) {
    if (c.ffn != DLM_FFN_MOE) return 0;
    return c.expert_dtype == DLM_MXFP4 ? 4 : c.expert_dtype == DLM_MXFP6 ? 6 : 0;
}

dlm_status check_weights(const dlm_config* c, const dlm_weights* w) {
    if (!w) return fail(DLM_E_ARG, "weights is NULL");
    if (!w->embed || !w->final_norm || !w->lm_head || !w->layers) return fail(DLM_E_ARG, "NULL top-level weight");
    const bool fp8 = c->dtype == DLM_FP8;
    if (fp8 && !w->lm_head_s) return fail(DLM_E_DTYPE, "fp8 model needs lm_head_s");
    for (int l = 0; l < c->n_layers; ++l) {
        const dlm_layer_weights& L = w->layers[l];
        if (!L.attn_norm || !L.ffn_norm || !L.wqkv || !L.wo || !L.w_gate || !L.w_up || !L.w_down)
            return fail(DLM_E_ARG, "layer %d: NULL weight", l);
        if (fp8 && (!L.wqkv_s || !L.wo_s || !L.w_gate_s || !L.w_up_s || !L.w_down_s))
            return fail(DLM_E_DTYPE, "layer %d: fp8 model needs per-channel scales", l);
        if (c->ffn == DLM_FFN_MOE) {
            if (!L.w_router || !L.we_gate || !L.we_up || !L.we_down)
                return fail(DLM_E_ARG, "layer %d: NULL expert weight", l);
            if (fp8 && (!L.we_gate_s || !L.we_up_s || !L.we_down_s))
                return fail(DLM_E_DTYPE, "layer %d: fp8 model needs expert scales", l);
            if (mx_bits(*c) && (!L.we_gate_e8 || !L.we_up_e8 || !L.we_down_e8))
                return fail(DLM_E_DTYPE, "layer %d: MX experts need their E8M0 scales", l);
        }
    }
    return DLM_OK;
}

dlm_status check_seq(const dlm_model* m, const dlm_seq* s, int extra, bool need_canvas, int idx) {
    if (!s) return fail(DLM_E_ARG, "seq %d is NULL", idx);
    if (!s->kv) return fail(DLM_E_ARG, "seq %d: kv is NULL", idx);
    if (s->page_table && s->page_size != KV_PAGE)
        return fail(DLM_E_UNSUPPORTED, "seq %d: page_size %d (pages hold %d tokens)", idx, s->page_size, KV_PAGE);
    if (!s->page_table && s->page_size) return fail(DLM_E_ARG, "seq %d: page_size without page_table", idx);
    if (s->page_table && s->capacity % KV_PAGE)
        return fail(DLM_E_SHAPE, "seq %d: paged capacity %d is not a multiple of %d", idx, s->capacity, KV_PAGE);
    if (need_canvas && !s->canvas) return fail(DLM_E_ARG, "seq %d: canvas is NULL", idx);
    if (s->T < 0 || s->capacity < 0) return fail(DLM_E_ARG, "seq %d: negative T or capacity", idx);
    if (s->capacity % 8 != 0) return fail(DLM_E_SHAPE, "seq %d: capacity %d is not a multiple of 8", idx, s->capacity);
    if ((long)s->T + extra > (long)s->capacity)
        return fail(DLM_E_CAPACITY, "seq %d: T %d + %d exceeds capacity %d", idx, s->T, extra, s->capacity);
    (void)m;
    return DLM_OK;
}

dlm_status check_ws(const dlm_model* m, void* ws, size_t ws_bytes, int rows, int max_kv) {
    if ((m->dbg_router || m->dbg_router_logits) && m->cfg.ffn == DLM_FFN_MOE &&
        (int64_t)m->cfg.n_layers * rows > m->dbg_cap)
        return fail(DLM_E_CAPACITY, "router debug buffers hold %lld (layer, row) pairs, the forward needs %lld",
                    (long long)m->dbg_cap, (long long)m->cfg.n_layers * rows);
    const size_t need = plan(m->cfg, rows, max_kv).total;
    if (!ws) return fail(DLM_E_WORKSPACE, "workspace is NULL");
    if (ws_bytes < need) return fail(DLM_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
    return DLM_OK;
}

dlm_status hip_status(const char* where) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(DLM_E_HIP, "%s: %s", where, hipGetErrorString(e));
    return DLM_OK;
}

// ---------------------------------------------------------------- forward --

enum Mode { PREFILL, DENOISE, APPEND };

// Runs a GEMM.  A split-K result is either summed right away by the split-K
// epilogue kernel, or -- when `consumed` -- handed back as Partials for the
// kernel that reads the result next (RMSNorm, RoPE, MoE combine) to sum.  An
// unsplit result is already applied (or stored in d.C).
Partials run_gemm(dlm_model* m, int id, const GemmDesc& d, hipStream_t st, bool consumed = false) {
    int splits;
    {
        Timed t(m, id, st);
        splits = gemm_main(d, st);
    }
    Partials out;
    if (splits <= 1) return out;
    if (consumed) {
        out.p = d.splitk;
        out.splits = splits;
        out.stride = (long)d.M * d.N;
        if (d.dtype == DT_FP8) {
            out.a_scale = d.a_scale;
            out.b_scale = d.b_scale;
        }
        return out;
    }
    Timed t(m, DLM_K_SPLITK_EPILOGUE, st);
    gemm_splitk_finish(d, splits, st);
    return out;
}

void forward(dlm_model* m, Mode mode, const SeqTab& seqs, const IdSource& ids, void* ws, float* conf, int* pred,
             float* logits, hipStream_t st) {
    const dlm_config& c = m->cfg;
    const int R = seqs.n * seqs.per_seq;
    int max_kv = 0;
    for (int i = 0; i < seqs.n; ++i) max_kv = std::max(max_kv, seqs.T[i] + seqs.per_seq);
    const Plan p = plan(c, R, max_kv);
    const bool f32 = c.dtype == DLM_F32, fp8 = c.dtype == DLM_FP8;
    const int d = c.d_model, qd = c.n_q_heads * c.head_dim;
    const int nqkv = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
    const int gdt = c.dtype;                       // GEMM operand type
    const int mxb = mx_bits(c);                    // MX routed experts: element bits (0: not MX)
    const bool mx = mxb != 0;
    float* x = at<float>(ws, p.x);
    void* hA = at<void>(ws, p.hA);
    uint8_t* hq = fp8 ? at<uint8_t>(ws, p.hq) : nullptr;
    float* hs = fp8 ? at<float>(ws, p.hs) : nullptr;
    float* qkv = at<float>(ws, p.qkv);
    void* q = at<void>(ws, p.q);
    void* ao = at<void>(ws, p.ao);
    void* fi = at<void>(ws, p.fi);
    Partials pending;                              // split residual update not yet added to x
    MoeGather pending_moe;                         // routed experts' output not yet added to x

    {
        Timed t(m, DLM_K_EMBED, st);
        embed(ids, R, m->w.embed, f32 ? DT_F32 : DT_BF16, d, c.vocab, c.mask_id, mode == APPEND, x, m->d_err, st);
    }

    // x += pending; RMSNorm into the GEMM operand: fp32 / bf16 in hA, fp8 also codes + scales
    auto norm = [&](const float* g) {
        Timed t(m, DLM_K_NORM, st);
        rmsnorm(x, pending, pending_moe, g, R, d, c.rms_eps, f32 ? (float*)hA : nullptr,
                f32 ? nullptr : (uint16_t*)hA, hq, hs, st);
        pending = Partials();
        pending_moe = MoeGather();
    };
    auto opA = [&](const void* bf, const void* q8) { return fp8 ? q8 : bf; };
    // a GEMM on stream s with split-K partials in region `part`
    auto dense_on = [&](hipStream_t s, size_t part, int id, GemmDesc g, bool consumed) {
        g.splitk = at<float>(ws, part);
        g.splitk_floats = p.splitk_floats;
        return run_gemm(m, id, g, s, consumed);
    };
    auto dense = [&](int id, GemmDesc g, bool consumed = false) { return dense_on(st, p.splitk, id, g, consumed); };
    auto quant_on = [&](hipStream_t s, const void* src, int rows, int cols, uint8_t* qd8, float* sc) {
        if (!fp8) return;
        Timed t(m, DLM_K_QUANT, s);
        quant_rows((const uint16_t*)src, rows, cols, qd8, sc, s);
    };
    auto quant = [&](const void* src, int rows, int cols, uint8_t* qd8, float* sc) {
        quant_on(st, src, rows, cols, qd8, sc);
    };

    for (int l = 0; l < c.n_layers; ++l) {
        const dlm_layer_weights& L = m->layers[l];
        norm(L.attn_norm);
        Partials qkv_res;
        {
            GemmDesc g;
            g.dtype = gdt; g.epi = GEMM_STORE_F32;
            g.A = opA(hA, hq); g.lda = d; g.a_scale = hs;
            g.B = L.wqkv; g.ldb = d; g.b_tiled = true; g.b_scale = L.wqkv_s;
            g.M = R; g.N = nqkv; g.K = d;
            g.C = qkv; g.ldc = nqkv;
            qkv_res = dense(DLM_K_GEMM_QKV, g, true);
            if (!qkv_res.p) qkv_res.p = qkv;
        }
        {
            Timed t(m, DLM_K_ROPE_KV, st);
            rope_kv(qkv_res, R, seqs, l, c.n_layers, c.n_q_heads, c.n_kv_heads, c.head_dim, c.rope_base, f32, q, st);
        }
        // Prefill and append produce the KV cache only: the last layer's
        // attention output, O projection and FFN feed nothing they return.
        if (mode != DENOISE && l == c.n_layers - 1) break;
        {
            Timed tm(m, DLM_K_ATTN_MERGE, st, false);   // handed to the split-KV merge launch
            Timed t(m, DLM_K_ATTN, st);
            AttnWork w{at<float>(ws, p.opart), at<float>(ws, p.mlpart), 0, tm.timer()};
            attention(q, seqs, l, c.n_layers, c.n_q_heads, c.n_kv_heads, c.head_dim, mode == PREFILL, f32, ao, w,
                      st);
        }
        quant(ao, R, qd, fp8 ? at<uint8_t>(ws, p.aoq) : nullptr, fp8 ? at<float>(ws, p.aos) : nullptr);
        {
            GemmDesc g;
            g.dtype = gdt; g.epi = GEMM_ADD_F32;
            g.A = opA(ao, fp8 ? at<uint8_t>(ws, p.aoq) : nullptr); g.lda = qd;
            g.a_scale = fp8 ? at<float>(ws, p.aos) : nullptr;
            g.B = L.wo; g.ldb = qd; g.b_tiled = true; g.b_scale = L.wo_s;
            g.M = R; g.N = d; g.K = qd;
            g.C = x; g.ldc = d;
            pending = dense(DLM_K_GEMM_O, g, true);
        }
        norm(L.ffn_norm);
        // dense SwiGLU FFN (the gate/up half), or the MoE's shared expert
        auto ffn_gate_up = [&](hipStream_t s, size_t part) {
            GemmDesc g;
            g.dtype = gdt; g.epi = GEMM_SWIGLU; g.out_f32 = f32;
            g.A = opA(hA, hq); g.lda = d; g.a_scale = hs;
            g.B = L.w_gate; g.B2 = L.w_up; g.ldb = d; g.b_tiled = true;
            g.b_scale = L.w_gate_s; g.b2_scale = L.w_up_s;
            g.M = R; g.N = c.d_ffn; g.K = d; g.C = fi; g.ldc = c.d_ffn;
            dense_on(s, part, DLM_K_GEMM_GATE_UP, g, false);
            quant_on(s, fi, R, c.d_ffn, fp8 ? at<uint8_t>(ws, p.fiq) : nullptr, fp8 ? at<float>(ws, p.fis) : nullptr);
        };
        // ... and its down half: x += result, or (consumed) split partials for the next reader
        auto ffn_down = [&](hipStream_t s, size_t part) {
            GemmDesc g;
            g.dtype = gdt; g.epi = GEMM_ADD_F32;
            g.A = opA(fi, fp8 ? at<uint8_t>(ws, p.fiq) : nullptr); g.lda = c.d_ffn;
            g.a_scale = fp8 ? at<float>(ws, p.fis) : nullptr;
            g.B = L.w_down; g.ldb = c.d_ffn; g.b_tiled = true; g.b_scale = L.w_down_s;
            g.M = R; g.N = d; g.K = c.d_ffn; g.C = x; g.ldc = d;
            return dense_on(s, part, DLM_K_GEMM_DOWN, g, true);
        };
        if (c.ffn == DLM_FFN_MOE) {
            // The shared expert goes to the side stream: it reads hA (or its
            // codes) and writes only fi (codes), its own split-K region and, if
            // unsplit, x -- which the main stream leaves alone until the join.
            // The routing chain reads hA too and writes only its own buffers.
            // (A failing event call leaves its error for hipGetLastError,
            // which the entry point reads after the forward.)
            Partials shared;
            (void)hipEventRecord(m->fork_ev, st);
            (void)hipStreamWaitEvent(m->side, m->fork_ev, 0);
            ffn_gate_up(m->side, p.splitk2);
            shared = ffn_down(m->side, p.splitk2);
            (void)hipEventRecord(m->join_ev, m->side);
            const int E = c.n_experts, k = c.top_k, De = c.d_expert, A = R * k;
            float* rl = at<float>(ws, p.rl);
            int* tid = at<int>(ws, p.tid);
            float* tw = at<float>(ws, p.tw);
            int* offs = at<int>(ws, p.offs);
            int* tstart = at<int>(ws, p.tstart);
            int* sorted = at<int>(ws, p.sorted);
            int* inv = at<int>(ws, p.inv);
            Partials router_logits;
            {
                GemmDesc g;   // router logits: bf16 operands (fp32 for f32 models), fp32 out
                g.dtype = f32 ? DT_F32 : DT_BF16; g.epi = GEMM_STORE_F32;
                g.A = hA; g.lda = d; g.B = L.w_router; g.ldb = d;
                g.M = R; g.N = E; g.K = d; g.C = rl; g.ldc = E;
                router_logits = dense(DLM_K_ROUTER, g, true);   // split partials are summed by the top-k
                if (!router_logits.p) router_logits.p = rl;
            }
            {
                Timed t(m, DLM_K_TOPK, st);
                router_topk(router_logits, R, E, k, tid, tw, m->dbg_router ? m->dbg_router + (long)l * R * k : nullptr,
                            m->dbg_router_logits ? m->dbg_router_logits + (long)l * R * E : nullptr, st);
            }
            {
                Timed t(m, DLM_K_PERMUTE, st);
                RouteWork rw{at<int>(ws, p.hist), at<int>(ws, p.lrank)};
                moe_route(tid, A, E, mx ? mx_grouped_bm() : grouped_bm(gdt, A, E), offs, tstart, sorted, inv, rw, st);
            }
            void* ei = at<void>(ws, p.ei);
            float* y = at<float>(ws, p.y);
            const bool y_bf16 = !mx && gdt == DT_BF16 && grouped_compute_bound(A, E);
            if (mx) {
                // MX experts: gate/up with the SwiGLU epilogue, then down, on
                // the bf16 activations
                MxDesc g;
                g.bits = mxb;
                g.swiglu = true;
                g.A = hA; g.lda = d; g.gather = sorted; g.gather_div = k;
                g.B = L.we_gate; g.B2 = L.we_up; g.S = L.we_gate_e8; g.S2 = L.we_up_e8;
                g.b_stride = mx_code_bytes(mxb, De, d); g.s_stride = mx_scale_bytes(De, d);
                g.offs = offs; g.tile_start = tstart; g.E = E;
                g.M = A; g.N = De; g.K = d; g.C = ei; g.ldc = De;
                {
                    Timed t(m, DLM_K_EXPERT_GATE_UP, st);
                    mx_grouped(g, st);
                }
                MxDesc h;
                h.bits = mxb;
                h.A = ei; h.lda = De;
                h.B = L.we_down; h.S = L.we_down_e8;
                h.b_stride = mx_code_bytes(mxb, d, De); h.s_stride = mx_scale_bytes(d, De);
                h.offs = offs; h.tile_start = tstart; h.E = E;
                h.M = A; h.N = d; h.K = De; h.C = y; h.ldc = d;
                Timed t(m, DLM_K_EXPERT_DOWN, st);
                mx_grouped(h, st);
            } else {
                {
                    GemmDesc g;
                    g.dtype = gdt; g.epi = GEMM_SWIGLU; g.out_f32 = f32;
                    g.A = opA(hA, hq); g.lda = d; g.a_scale = hs;
                    g.gather = sorted; g.gather_div = k;
                    g.B = L.we_gate; g.B2 = L.we_up; g.ldb = d; g.b_stride = packed_rows(De) * d; g.b_tiled = true;
                    g.b_scale = L.we_gate_s; g.b2_scale = L.we_up_s; g.bs_stride = De;
                    g.offs = offs; g.tile_start = tstart; g.E = E;
                    g.M = A; g.N = De; g.K = d; g.C = ei; g.ldc = De;
                    Timed t(m, DLM_K_EXPERT_GATE_UP, st);
                    gemm_grouped(g, st);
                }
                quant(ei, A, De, fp8 ? at<uint8_t>(ws, p.eiq) : nullptr, fp8 ? at<float>(ws, p.eis) : nullptr);
                // bf16 models with experts of 256 rows or more on average store
                // the per-assignment outputs in bf16: the combine, which reads
                // them once (weighted, into the fp32 residual stream), moves
                // half the bytes (32 requests: 6.6 -> 4.1 ms per step).  At a
                // canvas's ~16 rows per expert the combine is latency-bound
                // and the 2-byte epilogue stores cost more than they save.
                GemmDesc g;
                g.dtype = gdt; g.epi = y_bf16 ? GEMM_STORE_BF16 : GEMM_STORE_F32;
                g.A = opA(ei, fp8 ? at<uint8_t>(ws, p.eiq) : nullptr); g.lda = De;
                g.a_scale = fp8 ? at<float>(ws, p.eis) : nullptr;
                g.B = L.we_down; g.ldb = De; g.b_stride = packed_rows(d) * De; g.b_tiled = true;
                g.b_scale = L.we_down_s; g.bs_stride = d;
                g.offs = offs; g.tile_start = tstart; g.E = E;
                g.M = A; g.N = d; g.K = De; g.C = y; g.ldc = d;
                Timed t(m, DLM_K_EXPERT_DOWN, st);
                gemm_grouped(g, st);
            }
            (void)hipStreamWaitEvent(st, m->join_ev, 0);
            // x += shared + routed experts: added by the RMSNorm that reads x
            // next (the next layer's, or the final one); nothing touches x,
            // y, inv or the weights before it
            pending = shared;
            pending_moe = MoeGather{y, inv, tw, k, y_bf16};
        } else {
            ffn_gate_up(st, p.splitk);
            pending = ffn_down(st, p.splitk);
        }
    }
    if (mode != DENOISE) return;

    norm(m->w.final_norm);
    const int nt = (c.vocab + lm_head_tile_n(R) - 1) / lm_head_tile_n(R);
    float* pmax = at<float>(ws, p.pmax);
    float* psum = at<float>(ws, p.psum);
    int* pidx = at<int>(ws, p.pidx);
    {
        GemmDesc g;
        g.dtype = gdt; g.epi = GEMM_LMHEAD;
        g.A = opA(hA, hq); g.lda = d; g.a_scale = hs;
        g.B = m->w.lm_head; g.ldb = d; g.b_tiled = true; g.b_scale = m->w.lm_head_s;
        g.M = R; g.N = c.vocab; g.K = d;
        g.pmax = pmax; g.psum = psum; g.pidx = pidx; g.mask_col = c.mask_id;
        g.logits = logits; g.ld_logits = c.vocab;
        dense(DLM_K_LM_HEAD, g);
    }
    {
        Timed t(m, DLM_K_LM_MERGE, st);
        lm_merge(pmax, psum, pidx, R, nt, conf, pred, st);
    }
}

dlm_status build_tab(dlm_model* m, dlm_seq* const* seqs, int n_seqs, int extra, bool need_canvas, SeqTab& tab,
                     int& max_kv) {
    if (!seqs) return fail(DLM_E_ARG, "seqs is NULL");
    if (n_seqs < 1 || n_seqs > DLM_MAX_SEQS) return fail(DLM_E_ARG, "n_seqs %d not in [1, %d]", n_seqs, DLM_MAX_SEQS);
    memset(&tab, 0, sizeof tab);
    max_kv = 0;
    for (int i = 0; i < n_seqs; ++i) {
        dlm_status s = check_seq(m, seqs[i], extra, need_canvas, i);
        if (s) return s;
        tab.kv[i] = seqs[i]->kv;
        tab.pt[i] = seqs[i]->page_table;
        tab.T[i] = seqs[i]->T;
        tab.cap[i] = seqs[i]->capacity;
        max_kv = std::max(max_kv, seqs[i]->T + extra);
    }
    const dlm_config& c = m->cfg;
    tab.page_elems = (long)c.n_layers * 2 * c.n_kv_heads * KV_PAGE * c.head_dim;
    tab.n = n_seqs;
    tab.per_seq = extra;
    return DLM_OK;
}

}  // namespace

// ==================================================================== ABI ==

extern "C" {

const char* dlm_last_error(void) { return g_err.c_str(); }

const char* dlm_kernel_name(int32_t id) {
    return (id >= 0 && id < DLM_K_COUNT) ? kKernelNames[id] : "";
}

dlm_status dlm_create(const dlm_config* cfg, const dlm_weights* weights, dlm_model** out) {
    g_err.clear();
    if (!out) return fail(DLM_E_ARG, "out is NULL");
    *out = nullptr;
    dlm_status s = check_config(cfg);
    if (s) return s;
    s = check_weights(cfg, weights);
    if (s) return s;
    dlm_model* m = new dlm_model();
    m->cfg = *cfg;
    m->w = *weights;
    m->layers.assign(weights->layers, weights->layers + cfg->n_layers);
    m->w.layers = nullptr;
    hipError_t e = hipGetDevice(&m->device);
    if (e == hipSuccess) e = scratch_address(m->device, &m->scratch);
    if (e == hipSuccess) e = hipMalloc((void**)&m->d_err, sizeof(int));
    if (e == hipSuccess) e = hipMemset(m->d_err, 0, sizeof(int));
    if (e == hipSuccess && cfg->ffn == DLM_FFN_MOE) {
        e = hipStreamCreateWithFlags(&m->side, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&m->fork_ev, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&m->join_ev, hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        if (m->d_err) hipFree(m->d_err);
        if (m->fork_ev) (void)hipEventDestroy(m->fork_ev);
        if (m->join_ev) (void)hipEventDestroy(m->join_ev);
        if (m->side) (void)hipStreamDestroy(m->side);
        delete m;
        return fail(DLM_E_HIP, "dlm_create: %s", hipGetErrorString(e));
    }
    *out = m;
    return DLM_OK;
}

void dlm_destroy(dlm_model* m) {
    if (!m) return;
    for (auto& ev : m->pending) {
        hipEventDestroy(ev.a);
        hipEventDestroy(ev.b);
    }
    for (auto e : m->pool) hipEventDestroy(e);
    if (m->d_err) hipFree(m->d_err);
    if (m->fork_ev) (void)hipEventDestroy(m->fork_ev);
    if (m->join_ev) (void)hipEventDestroy(m->join_ev);
    if (m->side) (void)hipStreamDestroy(m->side);
    delete m;
}

size_t dlm_workspace_bytes(const dlm_model* m, int32_t max_rows, int32_t max_kv_tokens) {
    if (!m || max_rows < 1 || max_kv_tokens < 0) return 0;
    return plan(m->cfg, max_rows, max_kv_tokens).total;
}

dlm_status dlm_prefill(dlm_model* m, dlm_seq* seq, const int32_t* ids, int32_t n, void* ws, size_t ws_bytes,
                       void* stream) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    if (!ids) return fail(DLM_E_ARG, "ids is NULL");
    if (n < 1) return fail(DLM_E_ARG, "n %d < 1", n);
    SeqTab tab;
    int max_kv;
    dlm_seq* one[1] = {seq};
    dlm_status s = build_tab(m, one, 1, n, false, tab, max_kv);
    if (s) return s;
    s = check_ws(m, ws, ws_bytes, n, max_kv);
    if (s) return s;
    IdSource src{};
    src.flat = ids;
    src.per_seq = n;
    forward(m, PREFILL, tab, src, ws, nullptr, nullptr, nullptr, (hipStream_t)stream);
    s = hip_status("dlm_prefill");
    if (s) return s;
    seq->T += n;
    return DLM_OK;
}

dlm_status dlm_denoise_step(dlm_model* m, dlm_seq* const* seqs, int32_t n_seqs, float* conf, int32_t* pred,
                            float* logits, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    if (!conf || !pred) return fail(DLM_E_ARG, "conf / pred is NULL");
    SeqTab tab;
    int max_kv;
    dlm_status s = build_tab(m, seqs, n_seqs, m->cfg.canvas, true, tab, max_kv);
    if (s) return s;
    s = check_ws(m, ws, ws_bytes, n_seqs * m->cfg.canvas, max_kv);
    if (s) return s;
    IdSource src{};
    for (int i = 0; i < n_seqs; ++i) src.canvas[i] = seqs[i]->canvas;
    src.per_seq = m->cfg.canvas;
    forward(m, DENOISE, tab, src, ws, conf, pred, logits, (hipStream_t)stream);
    return hip_status("dlm_denoise_step");
}

dlm_status dlm_denoise_step_noalloc(dlm_model* m, dlm_seq* const* seqs, int32_t n_seqs, float* conf, int32_t* pred,
                                    float* logits, void* stream) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    if (!conf || !pred) return fail(DLM_E_ARG, "conf / pred is NULL");
    SeqTab tab;
    int max_kv;
    dlm_status s = build_tab(m, seqs, n_seqs, m->cfg.canvas, true, tab, max_kv);
    if (s) return s;
    const size_t need = plan(m->cfg, n_seqs * m->cfg.canvas, max_kv).total;
    if (need > DLM_STATIC_SCRATCH_BYTES)
        return fail(DLM_E_WORKSPACE, "the pass needs %zu bytes of workspace, the static scratch holds %zu", need,
                    (size_t)DLM_STATIC_SCRATCH_BYTES);
    s = check_ws(m, m->scratch, DLM_STATIC_SCRATCH_BYTES, n_seqs * m->cfg.canvas, max_kv);
    if (s) return s;
    IdSource src{};
    for (int i = 0; i < n_seqs; ++i) src.canvas[i] = seqs[i]->canvas;
    src.per_seq = m->cfg.canvas;
    forward(m, DENOISE, tab, src, m->scratch, conf, pred, logits, (hipStream_t)stream);
    return hip_status("dlm_denoise_step_noalloc");
}

dlm_status dlm_commit(dlm_model* m, dlm_seq* const* seqs, int32_t n_seqs, const float* conf, const int32_t* pred,
                      const dlm_commit_rule* rule, int32_t step, int32_t* n_committed, int32_t* n_masked,
                      void* stream) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    if (!conf || !pred) return fail(DLM_E_ARG, "conf / pred is NULL");
    if (!rule) return fail(DLM_E_ARG, "rule is NULL");
    if (!seqs) return fail(DLM_E_ARG, "seqs is NULL");
    if (n_seqs < 1 || n_seqs > DLM_MAX_SEQS) return fail(DLM_E_ARG, "n_seqs %d not in [1, %d]", n_seqs, DLM_MAX_SEQS);
    if (rule->n_steps < 1) return fail(DLM_E_ARG, "rule n_steps < 1");
    if (step < 0 || step >= rule->n_steps) return fail(DLM_E_ARG, "step %d outside [0, %d)", step, rule->n_steps);
    int kind, k = 0;
    bool force = false;
    if (rule->kind == DLM_COMMIT_TOPK) {
        if (!rule->k_per_step) return fail(DLM_E_ARG, "k_per_step is NULL");
        k = rule->k_per_step[step];
        if (k < 0) return fail(DLM_E_ARG, "k_per_step[%d] < 0", step);
        kind = 0;
    } else if (rule->kind == DLM_COMMIT_THRESHOLD) {
        if (!(rule->threshold >= 0.f)) return fail(DLM_E_ARG, "threshold must be >= 0");
        kind = 1;
        force = step == rule->n_steps - 1;
    } else {
        return fail(DLM_E_ARG, "unknown commit rule %d", rule->kind);
    }
    if (!(rule->edit_threshold >= 0.f) || !std::isfinite(rule->edit_threshold))
        return fail(DLM_E_ARG, "edit_threshold must be finite and >= 0");
    int32_t* canv[DLM_MAX_SEQS];
    for (int i = 0; i < n_seqs; ++i) {
        if (!seqs[i] || !seqs[i]->canvas) return fail(DLM_E_ARG, "seq %d: canvas is NULL", i);
        canv[i] = seqs[i]->canvas;
    }
    {
        Timed t(m, DLM_K_COMMIT, (hipStream_t)stream);
        commit(canv, n_seqs, m->cfg.canvas, conf, pred, m->cfg.mask_id, kind, k, rule->threshold, force,
               rule->edit_threshold, n_committed, n_masked, (hipStream_t)stream);
    }
    return hip_status("dlm_commit");
}

dlm_status dlm_append_canvas(dlm_model* m, dlm_seq* const* seqs, int32_t n_seqs, void* ws, size_t ws_bytes,
                             void* stream) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    SeqTab tab;
    int max_kv;
    dlm_status s = build_tab(m, seqs, n_seqs, m->cfg.canvas, true, tab, max_kv);
    if (s) return s;
    s = check_ws(m, ws, ws_bytes, n_seqs * m->cfg.canvas, max_kv);
    if (s) return s;
    IdSource src{};
    for (int i = 0; i < n_seqs; ++i) src.canvas[i] = seqs[i]->canvas;
    src.per_seq = m->cfg.canvas;
    forward(m, APPEND, tab, src, ws, nullptr, nullptr, nullptr, (hipStream_t)stream);
    s = hip_status("dlm_append_canvas");
    if (s) return s;
    for (int i = 0; i < n_seqs; ++i) seqs[i]->T += m->cfg.canvas;
    return DLM_OK;
}

dlm_status dlm_check_device_status(dlm_model* m, void* stream, int32_t* bits) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    int v = 0;
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e == hipSuccess) e = hipMemcpy(&v, m->d_err, sizeof(int), hipMemcpyDeviceToHost);
    if (e == hipSuccess && v) e = hipMemset(m->d_err, 0, sizeof(int));
    if (e != hipSuccess) return fail(DLM_E_HIP, "dlm_check_device_status: %s", hipGetErrorString(e));
    if (bits) *bits = v;
    if (v) return fail(DLM_E_DEVICE, "device error word 0x%x", v);
    return DLM_OK;
}

static GemmDesc op_gemm_desc(int32_t dtype, int32_t swiglu, int32_t M, int32_t N, int32_t K, int32_t variant,
                             int32_t splits) {
    GemmDesc g;
    g.dtype = dtype;
    g.epi = swiglu ? GEMM_SWIGLU : GEMM_STORE_F32;
    g.out_f32 = dtype == DLM_F32;
    g.M = M; g.N = N; g.K = K;
    g.lda = K; g.ldb = K; g.ldc = N;
    g.variant = variant & 0xff;
    g.b_tiled = (variant & DLM_GEMM_B_TILED) != 0;
    g.force_splits = splits;
    return g;
}

static dlm_status op_gemm_check(int32_t dtype, int32_t M, int32_t N, int32_t K, int32_t variant, int32_t splits) {
    if (dtype != DLM_F32 && dtype != DLM_BF16 && dtype != DLM_FP8) return fail(DLM_E_UNSUPPORTED, "dtype %d", dtype);
    if (M < 1 || N < 1 || K < 1) return fail(DLM_E_ARG, "M, N, K must be >= 1");
    if (((long)K * elem_bytes(dtype)) % 128) return fail(DLM_E_SHAPE, "K * element size not a multiple of 128");
    if (variant < 0 || (variant & ~(0xff | DLM_GEMM_B_TILED)) || (variant & 0xff) > gemm_variants())
        return fail(DLM_E_ARG, "variant %d", variant);
    if (splits < 0) return fail(DLM_E_ARG, "splits %d", splits);
    return DLM_OK;
}

static dlm_status pack_check(int32_t dtype, int32_t batch, int32_t N, int32_t K) {
    if (dtype != DLM_F32 && dtype != DLM_BF16 && dtype != DLM_FP8) return fail(DLM_E_DTYPE, "dtype %d", dtype);
    if (batch < 1 || N < 1 || K < 1) return fail(DLM_E_ARG, "batch / N / K < 1");
    if (((long)K * elem_bytes(dtype)) % 128) return fail(DLM_E_SHAPE, "K * element size not a multiple of 128");
    return DLM_OK;
}

size_t dlm_packed_weight_bytes(int32_t dtype, int32_t batch, int32_t N, int32_t K) {
    if (pack_check(dtype, batch, N, K)) return 0;
    return (size_t)packed_weight_bytes(elem_bytes(dtype), batch, N, K);
}

dlm_status dlm_pack_weight(int32_t dtype, int32_t batch, int32_t N, int32_t K, const void* src, void* dst,
                           void* stream) {
    g_err.clear();
    dlm_status s = pack_check(dtype, batch, N, K);
    if (s) return s;
    if (!src || !dst) return fail(DLM_E_ARG, "null pointer");
    const uintptr_t a0 = (uintptr_t)src, a1 = a0 + (size_t)batch * N * K * elem_bytes(dtype);
    const uintptr_t b0 = (uintptr_t)dst, b1 = b0 + (size_t)packed_weight_bytes(elem_bytes(dtype), batch, N, K);
    if (a0 < b1 && b0 < a1) return fail(DLM_E_ARG, "src and dst overlap");
    pack_weight(elem_bytes(dtype), batch, N, K, src, dst, (hipStream_t)stream);
    return hip_status("dlm_pack_weight");
}

static int mx_dtype_bits(int32_t dtype) { return dtype == DLM_MXFP4 ? 4 : dtype == DLM_MXFP6 ? 6 : 0; }

static dlm_status mx_check(int32_t dtype, int32_t batch, int32_t N, int32_t K) {
    if (!mx_dtype_bits(dtype)) return fail(DLM_E_DTYPE, "dtype %d is not an MX format", dtype);
    if (batch < 1 || N < 1 || K < 1) return fail(DLM_E_ARG, "batch / N / K < 1");
    if (K % 128) return fail(DLM_E_SHAPE, "K %d is not a multiple of 128", K);
    return DLM_OK;
}

size_t dlm_packed_mx_bytes(int32_t dtype, int32_t batch, int32_t N, int32_t K, int32_t scales) {
    if (mx_check(dtype, batch, N, K)) return 0;
    return (size_t)batch * (size_t)(scales ? mx_scale_bytes(N, K) : mx_code_bytes(mx_dtype_bits(dtype), N, K));
}

dlm_status dlm_pack_mx(int32_t dtype, int32_t batch, int32_t N, int32_t K, const void* codes, const void* scales,
                       void* dst_codes, void* dst_scales, void* stream) {
    g_err.clear();
    dlm_status s = mx_check(dtype, batch, N, K);
    if (s) return s;
    if (!codes || !scales || !dst_codes || !dst_scales) return fail(DLM_E_ARG, "null pointer");
    if (((uintptr_t)codes | (uintptr_t)dst_codes) % 16) return fail(DLM_E_ARG, "codes not 16-byte aligned");
    struct Range { uintptr_t lo, hi; };
    const Range r[4] = {
        {(uintptr_t)codes, (uintptr_t)codes + (size_t)batch * N * ((size_t)K * mx_dtype_bits(dtype) / 8)},
        {(uintptr_t)scales, (uintptr_t)scales + (size_t)batch * N * (K / 32)},
        {(uintptr_t)dst_codes, (uintptr_t)dst_codes + dlm_packed_mx_bytes(dtype, batch, N, K, 0)},
        {(uintptr_t)dst_scales, (uintptr_t)dst_scales + dlm_packed_mx_bytes(dtype, batch, N, K, 1)}};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if ((i >= 2 || j >= 2) && r[i].lo < r[j].hi && r[j].lo < r[i].hi)
                return fail(DLM_E_ARG, "packed output overlaps another buffer");
    mx_pack(mx_dtype_bits(dtype), batch, N, K, codes, scales, dst_codes, dst_scales, (hipStream_t)stream);
    return hip_status("dlm_pack_mx");
}

size_t dlm_op_mx_gemm_workspace(int32_t E) {
    if (E < 1 || E > 256) return 0;
    return 2 * align_up((size_t)(E + 1) * 4);
}

dlm_status dlm_op_mx_gemm(int32_t dtype, int32_t swiglu, int32_t E, const int32_t* counts, int32_t N, int32_t K,
                          const void* A, const void* B, const void* S, const void* B2, const void* S2, void* C,
                          void* ws, size_t ws_bytes, int32_t variant, float* ms, void* stream) {
    g_err.clear();
    if (!mx_dtype_bits(dtype)) return fail(DLM_E_DTYPE, "dtype %d is not an MX format", dtype);
    if (!counts || !A || !B || !S || !C || !ws || (swiglu && (!B2 || !S2))) return fail(DLM_E_ARG, "null pointer");
    if (E < 1 || E > 256) return fail(DLM_E_ARG, "E %d not in [1, 256]", E);
    if (variant < 0 || variant > mx_variants()) return fail(DLM_E_ARG, "variant %d not in 0..%d", variant, mx_variants());
    if (N < 1 || K < 1 || K % 128) return fail(DLM_E_SHAPE, "N %d, K %d (K a multiple of 128)", N, K);
    if (ws_bytes < dlm_op_mx_gemm_workspace(E)) return fail(DLM_E_WORKSPACE, "workspace %zu bytes too small", ws_bytes);
    // the routing's offsets and m-tile starts for these counts
    std::vector<int32_t> host(2 * (E + 1));
    long M = 0, tiles = 0;
    const int bm = mx_grouped_bm();
    for (int e = 0; e < E; ++e) {
        if (counts[e] < 0) return fail(DLM_E_ARG, "counts[%d] = %d < 0", e, counts[e]);
        host[e] = (int32_t)M;
        host[E + 1 + e] = (int32_t)tiles;
        M += counts[e];
        tiles += (counts[e] + bm - 1) / bm;
        if (M > (1 << 24)) return fail(DLM_E_ARG, "more than 2^24 rows");
    }
    if (M < 1) return fail(DLM_E_ARG, "no rows");
    host[E] = (int32_t)M;
    host[2 * E + 1] = (int32_t)tiles;
    hipStream_t st = (hipStream_t)stream;
    int* offs = at<int>(ws, 0);
    int* tstart = at<int>(ws, align_up((size_t)(E + 1) * 4));
    hipError_t e = hipMemcpyAsync(offs, host.data(), (size_t)(E + 1) * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(tstart, host.data() + E + 1, (size_t)(E + 1) * 4, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);   // `host` dies with this call
    if (e != hipSuccess) return fail(DLM_E_HIP, "dlm_op_mx_gemm: %s", hipGetErrorString(e));
    MxDesc d;
    d.bits = mx_dtype_bits(dtype);
    d.swiglu = swiglu != 0;
    d.A = A; d.lda = K;
    d.B = B; d.B2 = B2; d.S = S; d.S2 = S2;
    d.b_stride = mx_code_bytes(d.bits, N, K); d.s_stride = mx_scale_bytes(N, K);
    d.offs = offs; d.tile_start = tstart; d.E = E;
    d.M = (int)M; d.N = N; d.K = K; d.C = C; d.ldc = N;
    d.variant = variant;
    LaunchTimer lt;
    if (ms) {
        hipEventCreate(&lt.start);
        hipEventCreate(&lt.stop);
        lt.armed = true;
        launch_timer() = &lt;
    }
    mx_grouped(d, st);
    launch_timer() = nullptr;
    dlm_status s = hip_status("dlm_op_mx_gemm");
    if (ms) {
        if (!s) {
            e = hipEventSynchronize(lt.stop);
            if (e == hipSuccess) e = hipEventElapsedTime(ms, lt.start, lt.stop);
            if (e != hipSuccess) s = fail(DLM_E_HIP, "dlm_op_mx_gemm timing: %s", hipGetErrorString(e));
        }
        hipEventDestroy(lt.start);
        hipEventDestroy(lt.stop);
    }
    return s;
}

size_t dlm_op_gemm_workspace(int32_t dtype, int32_t swiglu, int32_t M, int32_t N, int32_t K, int32_t variant,
                             int32_t splits) {
    if (op_gemm_check(dtype, M, N, K, variant, splits)) return 0;
    return (size_t)gemm_splitk_floats(op_gemm_desc(dtype, swiglu, M, N, K, variant, splits)) * 4;
}

dlm_status dlm_op_gemm(int32_t dtype, int32_t swiglu, int32_t M, int32_t N, int32_t K, const void* A, const void* B,
                       const void* B2, const float* a_scale, const float* b_scale, const float* b2_scale, void* C,
                       void* ws, size_t ws_bytes, int32_t variant, int32_t splits, float* ms, void* stream) {
    g_err.clear();
    dlm_status s = op_gemm_check(dtype, M, N, K, variant, splits);
    if (s) return s;
    if (!A || !B || !C || (swiglu && !B2)) return fail(DLM_E_ARG, "null pointer");
    if (dtype == DLM_FP8 && (!a_scale || !b_scale || (swiglu && !b2_scale)))
        return fail(DLM_E_ARG, "fp8 needs a_scale, b_scale (and b2_scale)");
    GemmDesc g = op_gemm_desc(dtype, swiglu, M, N, K, variant, splits);
    g.a_scale = a_scale; g.b_scale = b_scale; g.b2_scale = b2_scale;
    const long need = gemm_splitk_floats(g);
    if (need > 0 && (!ws || ws_bytes < (size_t)need * 4))
        return fail(DLM_E_WORKSPACE, "split-K needs %ld bytes", need * 4);
    g.A = A; g.B = B; g.B2 = B2; g.C = C;
    g.splitk = (float*)ws;
    g.splitk_floats = (long)(ws_bytes / 4);
    hipStream_t st = (hipStream_t)stream;
    LaunchTimer lt;
    if (ms) {
        hipEventCreate(&lt.start);
        hipEventCreate(&lt.stop);
        lt.armed = true;
        launch_timer() = &lt;
    }
    const int used = gemm_main(g, st);
    launch_timer() = nullptr;
    if (used > 1) gemm_splitk_finish(g, used, st);
    s = hip_status("dlm_op_gemm");
    if (ms) {
        if (!s) {
            hipError_t e = hipEventSynchronize(lt.stop);
            if (e == hipSuccess) e = hipEventElapsedTime(ms, lt.start, lt.stop);
            if (e != hipSuccess) s = fail(DLM_E_HIP, "dlm_op_gemm timing: %s", hipGetErrorString(e));
        }
        hipEventDestroy(lt.start);
        hipEventDestroy(lt.stop);
    }
    return s;
}

dlm_status dlm_op_quant_rows(const void* x, int32_t rows, int32_t d, void* q, float* s, void* stream) {
    g_err.clear();
    if (!x || !q || !s) return fail(DLM_E_ARG, "null pointer");
    if (rows < 1 || d < 1) return fail(DLM_E_ARG, "rows and d must be >= 1");
    quant_rows((const uint16_t*)x, rows, d, (uint8_t*)q, s, (hipStream_t)stream);
    return hip_status("dlm_op_quant_rows");
}

// Workspace of dlm_op_route: the ids, then the multi-kernel path's block
// histograms and local ranks, each 256-byte aligned.
static size_t route_ws_layout(int32_t n_assign, int32_t E, size_t* hist_off, size_t* rank_off) {
    const size_t ids = align_up((size_t)n_assign * 4);
    const size_t hist = align_up((size_t)route_blocks(n_assign) * E * 4);
    if (hist_off) *hist_off = ids;
    if (rank_off) *rank_off = ids + hist;
    return ids + hist + align_up((size_t)n_assign * 4);
}

size_t dlm_op_route_workspace(int32_t n_assign, int32_t E) {
    if (n_assign < 1 || E < 1 || E > 256) return 0;
    return route_ws_layout(n_assign, E, nullptr, nullptr);
}

dlm_status dlm_op_route(const int32_t* ids, int32_t n_assign, int32_t E, int32_t bm, int32_t* offs, int32_t* tile_start,
                        int32_t* sorted_assign, int32_t* inv, void* ws, size_t ws_bytes, void* stream) {
    g_err.clear();
    if (!ids || !offs || !tile_start || !sorted_assign || !inv || !ws) return fail(DLM_E_ARG, "null pointer");
    if (n_assign < 1) return fail(DLM_E_ARG, "n_assign %d < 1", n_assign);
    if (E < 1 || E > 256) return fail(DLM_E_ARG, "E %d not in [1, 256]", E);
    if (bm < 1) return fail(DLM_E_ARG, "bm %d < 1", bm);
    for (int32_t a = 0; a < n_assign; ++a)
        if (ids[a] < 0 || ids[a] >= E) return fail(DLM_E_ARG, "ids[%d] = %d outside [0, %d)", a, ids[a], E);
    size_t hist_off, rank_off;
    const size_t need = route_ws_layout(n_assign, E, &hist_off, &rank_off);
    if (ws_bytes < need) return fail(DLM_E_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
    hipStream_t st = (hipStream_t)stream;
    int* d_ids = at<int>(ws, 0);
    hipError_t e = hipMemcpyAsync(d_ids, ids, (size_t)n_assign * 4, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return fail(DLM_E_HIP, "dlm_op_route: %s", hipGetErrorString(e));
    RouteWork rw{at<int>(ws, hist_off), at<int>(ws, rank_off)};
    moe_route(d_ids, n_assign, E, bm, offs, tile_start, sorted_assign, inv, rw, st);
    return hip_status("dlm_op_route");
}

dlm_status dlm_op_router_topk(const float* logits, int32_t rows, int32_t E, int32_t k, int32_t* ids, float* w,
                              void* stream) {
    g_err.clear();
    if (!logits || !ids || !w) return fail(DLM_E_ARG, "null pointer");
    if (rows < 1) return fail(DLM_E_ARG, "rows %d < 1", rows);
    if (E < 1 || E > 256) return fail(DLM_E_ARG, "E %d not in [1, 256]", E);
    if (k < 1 || k > 16 || k > E) return fail(DLM_E_ARG, "k %d not in [1, min(16, E)]", k);
    Partials p;
    p.p = logits;
    router_topk(p, rows, E, k, ids, w, nullptr, nullptr, (hipStream_t)stream);
    return hip_status("dlm_op_router_topk");
}

dlm_status dlm_debug_router(dlm_model* m, int32_t* router_ids, float* router_logits, int64_t capacity_rows) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    if ((router_ids || router_logits) && capacity_rows < 0) return fail(DLM_E_ARG, "negative capacity");
    m->dbg_router = router_ids;
    m->dbg_router_logits = router_logits;
    m->dbg_cap = (router_ids || router_logits) ? capacity_rows : 0;
    return DLM_OK;
}

dlm_status dlm_timing_enable(dlm_model* m, int32_t mask) {
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    m->timing_mask = (uint32_t)mask;
    return DLM_OK;
}

dlm_status dlm_timing_read(dlm_model* m, float* ms, int32_t* launches) {
    g_err.clear();
    if (!m) return fail(DLM_E_ARG, "model is NULL");
    for (auto& ev : m->pending) {
        hipError_t e = hipEventSynchronize(ev.b);
        float t = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, ev.a, ev.b);
        if (e != hipSuccess) return fail(DLM_E_HIP, "dlm_timing_read: %s", hipGetErrorString(e));
        m->ms[ev.id] += t;
        m->launches[ev.id] += 1;
        m->pool.push_back(ev.a);
        m->pool.push_back(ev.b);
    }
    m->pending.clear();
    for (int i = 0; i < DLM_K_COUNT; ++i) {
        if (ms) ms[i] = m->ms[i];
        if (launches) launches[i] = m->launches[i];
        m->ms[i] = 0.f;
        m->launches[i] = 0;
    }
    return DLM_OK;
}

}  // extern "C"
