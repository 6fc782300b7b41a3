// C ABI of the library: argument validation, workspace layout, the layer's
// step loop and HIP-graph plans. Declarations and semantics: include/rt_prefill.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "rt_internal.h"

namespace {

thread_local std::string g_last_error;

rt_status fail(rt_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

rt_status hip_fail(hipError_t e, const char* what) {
    return fail(RT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t elem_bytes(rt_dtype dt) { return dt == RT_BF16 ? 2 : 4; }

// Largest power of two dividing t (t >= 1): the block size of step t
// (reading note lshu.cn/news/403416, summary section 4.2).
int32_t block_of(int32_t t) { return t & -t; }

rt_status check_attn(const rt_attn_desc* d) {
    if (!d) return fail(RT_ERR_INVALID_ARG, "descriptor is NULL");
    if (d->batch <= 0 || d->seq_len <= 0 || d->n_heads <= 0 || d->head_dim <= 0)
        return fail(RT_ERR_INVALID_ARG, "batch, seq_len, n_heads and head_dim must be positive");
    if (d->dtype != RT_F32 && d->dtype != RT_BF16) return fail(RT_ERR_INVALID_ARG, "unknown dtype %d", (int)d->dtype);
    if (d->head_dim != 32 && d->head_dim != 64 && d->head_dim != 128)
        return fail(RT_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64 or 128)", d->head_dim);
    if (!std::isfinite(d->softmax_scale) || d->softmax_scale < 0.f)
        return fail(RT_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
    const double elems = (double)d->batch * d->seq_len * d->n_heads * d->head_dim;
    if (elems > 4.0e12) return fail(RT_ERR_UNSUPPORTED, "tensor too large");
    return RT_OK;
}

rt_status check_layer(const rt_layer_desc* d) {
    if (!d) return fail(RT_ERR_INVALID_ARG, "descriptor is NULL");
    rt_status st = check_attn(&d->attn);
    if (st != RT_OK) return st;
    if (d->d_model != d->attn.n_heads * d->attn.head_dim)
        return fail(RT_ERR_INVALID_ARG, "d_model %d != n_heads*head_dim %d", d->d_model,
                    d->attn.n_heads * d->attn.head_dim);
    if (d->d_ff <= 0) return fail(RT_ERR_INVALID_ARG, "d_ff must be positive");
    if (!(d->rms_eps >= 0.f) || !std::isfinite(d->rms_eps)) return fail(RT_ERR_INVALID_ARG, "rms_eps must be >= 0");
    if (!std::isfinite(d->residual_scale)) return fail(RT_ERR_INVALID_ARG, "residual_scale must be finite");
    if (d->attn.dtype == RT_BF16 && (d->d_model % 128 || d->d_ff % 128))
        return fail(RT_ERR_UNSUPPORTED, "bf16 layers need d_model and d_ff multiples of 128");
    if ((d->flags & RT_FLAG_NAIVE_SCHEDULE) && (d->flags & RT_FLAG_TRANSFORMER))
        return fail(RT_ERR_INVALID_ARG, "RT_FLAG_NAIVE_SCHEDULE and RT_FLAG_TRANSFORMER exclude each other");
    if (d->flags & ~(RT_FLAG_DEBUG_SYNC | RT_FLAG_NAIVE_SCHEDULE | RT_FLAG_TRANSFORMER | RT_FLAG_QK_NORM))
        return fail(RT_ERR_INVALID_ARG, "unknown flags 0x%x", d->flags);
    if ((d->flags & RT_FLAG_QK_NORM) && d->attn.dtype == RT_BF16 && d->attn.head_dim > 64)
        return fail(RT_ERR_UNSUPPORTED, "the bf16 query/key norm supports head_dim 32 or 64");
    if (d->attn.dtype == RT_BF16 && d->d_model > 64 * rt::kRowSSTile)
        return fail(RT_ERR_UNSUPPORTED, "bf16 layers support d_model up to %d", 64 * rt::kRowSSTile);
    if (d->kv_source_norm != 0 && d->kv_source_norm != 1)
        return fail(RT_ERR_INVALID_ARG, "kv_source_norm must be 0 or 1 (got %d)", d->kv_source_norm);
    if (!d->kv_source_norm && (d->flags & RT_FLAG_TRANSFORMER))
        return fail(RT_ERR_INVALID_ARG, "the Transformer layer's pair is its ephemeral pair: kv_source_norm must be 1");
    return RT_OK;
}

// What a workspace is laid out for.
enum class Mode {
    Blocked,      // RT layer, blocked schedule (the default)
    Naive,        // RT layer, naive schedule: position t's query reads pairs 1..t-1 in one pass
    Transformer,  // standard layer: pairs from the input, every position at once
    Decode,       // one RT (or Transformer) position against a cache
};

Mode mode_of(const rt_layer_desc* d) {
    if (d->flags & RT_FLAG_TRANSFORMER) return Mode::Transformer;
    if (d->flags & RT_FLAG_NAIVE_SCHEDULE) return Mode::Naive;
    return Mode::Blocked;
}

// Workspace layout of one layer forward (byte offsets, 256-aligned).
// Sizes below are for the blocked schedule; "rows" is B for the modes that
// run position by position and N*B for the Transformer layer.
struct Layout {
    size_t q, ke, ve;     // [N][B][d] dtype: queries and ephemeral pairs, formed up front
    size_t m, l, o;       // [N][B][H], [N][B][H], [N][B][H][dh] fp32: online-softmax state (blocked only)
    size_t a;             // [rows][d] dtype: attention output
    size_t h;             // [rows][d] fp32: residual stream after the attention branch
    size_t g;             // [rows][F] dtype: MLP hidden activation
    size_t hb;            // [rows][d] bf16: h rounded, the MLP's first operand (bf16 layers)
    size_t hss, zss;      // [rows][d/32] fp32: partial row sums of h^2 and of z^2 (bf16 layers)
    size_t wq, wk, wv, w1;// gain-folded weights (used when gains are given; bf16: two halves per row)
    size_t xss;           // [N*B][4] fp32: quarter-row sums of x^2 (bf16 layers: the up-front RMS)
    size_t total;
};

Layout layout_of(const rt_layer_desc* d, Mode mode) {
    const size_t es = elem_bytes(d->attn.dtype);
    const size_t N = mode == Mode::Decode ? 1 : d->attn.seq_len;
    const size_t B = d->attn.batch, H = d->attn.n_heads, D = d->d_model, F = d->d_ff;
    const size_t rows = mode == Mode::Transformer ? N * B : B;
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    L.q = take(N * B * D * es);
    if (mode != Mode::Transformer) {  // (the Transformer's pairs go straight into the caches)
        L.ke = take(N * B * D * es);
        L.ve = take(N * B * D * es);
    }
    if (mode == Mode::Blocked) {
        L.m = take(N * B * H * 4);
        L.l = take(N * B * H * 4);
        L.o = take(N * B * D * 4);
    }
    L.a = take(rows * D * es);
    L.h = take(rows * D * 4);
    L.g = take(rows * F * es);
    L.hb = take(rows * D * 2);
    L.hss = take(D / rt::kRowSSTile * rows * 4 + 4);
    L.zss = take(D / rt::kRowSSTile * rows * 4 + 4);
    const size_t halves = d->attn.dtype == RT_BF16 ? 2 : 1;  // a bf16 folded weight is stored in two halves
    L.wq = take(halves * D * D * es);
    L.wk = take(halves * D * D * es);
    L.wv = take(halves * D * D * es);
    L.w1 = take(halves * F * D * es);
    L.xss = take(N * B * 16);
    L.total = off;
    return L;
}

// A capture in progress on this thread (plans): the launches are recorded
// into graphs of at most `limit` launches each, ended and begun again on the
// capture stream (one graph with ~10^5 nodes of a long sequence did not
// survive instantiation; a chain of graphs replays the same launches in order).
struct CaptureSegments {
    hipStream_t s;
    int limit = 8192;
    int count = 0;
    std::vector<hipGraph_t> graphs;
    rt_status cut() {
        hipGraph_t g = nullptr;
        hipError_t e = hipStreamEndCapture(s, &g);
        if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
        graphs.push_back(g);
        e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
        count = 0;
        return RT_OK;
    }
};
thread_local CaptureSegments* g_capture = nullptr;

struct Launcher {
    hipStream_t s;
    bool debug;
    rt_status check(hipError_t e, const char* what) {
        if (e != hipSuccess) return hip_fail(e, what);
        if (debug) {
            e = hipStreamSynchronize(s);
            if (e != hipSuccess) return hip_fail(e, what);
        }
        if (g_capture && g_capture->s == s && ++g_capture->count >= g_capture->limit) return g_capture->cut();
        return RT_OK;
    }
};

#define RT_TRY(expr)                    \
    do {                                \
        rt_status _st = (expr);         \
        if (_st != RT_OK) return _st;   \
    } while (0)

rt_status check_layer_ptrs(const rt_layer_weights* w, const void* x, void* z, void* kc, void* vc, void* ws) {
    if (!w) return fail(RT_ERR_INVALID_ARG, "weights is NULL");
    const void* ps[] = {w->w_q, w->w_k, w->w_v, w->w_o, w->w_1, w->w_2, x, z, kc, vc, ws};
    const char* names[] = {"w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "x", "z", "k_cache", "v_cache", "workspace"};
    for (int i = 0; i < 11; ++i) {
        if (!ps[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned16(ps[i])) return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (((uintptr_t)ws & 255u) != 0) return fail(RT_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if ((w->g_attn && !aligned16(w->g_attn)) || (w->g_mlp && !aligned16(w->g_mlp)) ||
        (w->g_q && !aligned16(w->g_q)) || (w->g_k && !aligned16(w->g_k)))
        return fail(RT_ERR_INVALID_ARG, "gains must be 16-byte aligned");
    return RT_OK;
}

// The projections each RMS normalisation feeds, with the gain folded in
// (W'[r][c] = W[r][c] g[c]) when a gain is given. A bf16 folded weight holds
// two bf16 halves per row (launch_fold_gain), so its products run over
// kq (or k1) = 2 d columns, each A row read twice.
struct Projections {
    const void *wq, *wk, *wv, *w1;
    int32_t kq, k1;  // K of the products with W_q, W_k, W_v and with W_1
};

rt_status enqueue_fold(const rt_layer_desc* d, const rt_layer_weights* w, char* base, const Layout& L,
                       Launcher& run, Projections* p) {
    using namespace rt;
    const rt_dtype dt = d->attn.dtype;
    const int32_t D = d->d_model, F = d->d_ff;
    hipStream_t s = run.s;
    const int32_t halves = dt == RT_BF16 ? 2 : 1;
    *p = Projections{w->w_q, w->w_k, w->w_v, w->w_1, D, D};
    if (w->g_attn) {
        RT_TRY(run.check(launch_fold_gain(dt, w->w_q, w->g_attn, base + L.wq, D, D, s), "fold g_attn"));
        RT_TRY(run.check(launch_fold_gain(dt, w->w_k, w->g_attn, base + L.wk, D, D, s), "fold g_attn"));
        RT_TRY(run.check(launch_fold_gain(dt, w->w_v, w->g_attn, base + L.wv, D, D, s), "fold g_attn"));
        p->wq = base + L.wq;
        p->wk = base + L.wk;
        p->wv = base + L.wv;
        p->kq = halves * D;
    }
    if (w->g_mlp) {
        RT_TRY(run.check(launch_fold_gain(dt, w->w_1, w->g_mlp, base + L.w1, F, D, s), "fold g_mlp"));
        p->w1 = base + L.w1;
        p->k1 = halves * D;
    }
    return RT_OK;
}

// The product q | k' | v' = W_{q,k,v} RMS_attn(x) for `rows` rows of x (with
// the query/key norm on q and k' when the layer has it); bf16 layers take the
// RMS from the rows' quarter sums of squares in xss.
rt::GemmArgs qkv_args(const rt_layer_desc* d, const rt_layer_weights* w, const Projections& p, const void* x,
                      int64_t rows, void* q, void* ke, void* ve, const float* xss) {
    using namespace rt;
    const int32_t D = d->d_model;
    GemmArgs gq{};
    if (d->attn.dtype == RT_BF16) {
        gq.rss_in = xss; gq.n_parts = 4;
    }
    gq.A = x; gq.lda = D;
    gq.W[0] = p.wq; gq.W[1] = p.wk; gq.W[2] = p.wv;
    gq.C[0] = q; gq.C[1] = ke; gq.C[2] = ve;
    gq.ldc = D; gq.seg_n = D; gq.eps = d->rms_eps;
    gq.M = rows; gq.N = 3 * D; gq.K = p.kq; gq.a_k = D;
    if (d->flags & RT_FLAG_QK_NORM) {
        gq.qkn_mask = 3; gq.head_dim = d->attn.head_dim;
        gq.qkn_gain[0] = w->g_q; gq.qkn_gain[1] = w->g_k;
    }
    return gq;
}

// q | k' | v' for `rows` rows of x.
rt_status enqueue_qkv(const rt_layer_desc* d, const rt_layer_weights* w, const Projections& p, const void* x,
                      int64_t rows, void* q, void* ke, void* ve, float* xss, Launcher& run) {
    using namespace rt;
    if (d->attn.dtype == RT_BF16)
        // the rows' sums of squares in a pass of their own: summing them inside the
        // product's K loop (on the waves holding A) measured 15 % slower at N*B rows
        RT_TRY(run.check(launch_row_sumsq(RT_BF16, x, rows, d->d_model, xss, run.s), "row sums of squares"));
    const GemmArgs gq = qkv_args(d, w, p, x, rows, q, ke, ve, xss);
    return run.check(launch_gemm(d->attn.dtype, GemmKind::QKV, gq, run.s), "qkv projection");
}

// The products after the attention, for `rows` rows:
//   h = x + rho W_o a;  z = h + rho W_2 GELU(W_1 RMS_mlp(h));
//   and, when kt is not NULL, the persistent pair k|v = W_{k,v} RMS_attn(z).
// bf16 layers: W_o also stores h rounded to bf16 (the MLP's operand) and
// per-row partial sums of h^2; W_2 stores partial sums of z^2 (z as stored).
// The next product turns those sums into its RMS row scale.
struct TailArgs {
    rt::GemmArgs wo, w1, w2, kv;
};

TailArgs tail_args(const rt_layer_desc* d, const rt_layer_weights* w, const Projections& p, char* base,
                   const Layout& L, int64_t rows, const void* a, const void* x, void* z, void* kt, void* vt) {
    using namespace rt;
    const rt_dtype dt = d->attn.dtype;
    const int32_t D = d->d_model, F = d->d_ff;
    void* g = base + L.g;
    float* h = (float*)(base + L.h);
    const bool b16 = dt == RT_BF16;
    const int32_t parts = D / kRowSSTile;
    TailArgs ta{};

    GemmArgs& go = ta.wo;  // h = x + rho W_o a
    go.A = a; go.lda = D; go.W[0] = w->w_o; go.C[0] = h; go.ldc = D; go.seg_n = D;
    go.R = x; go.ldr = D; go.rscale = d->residual_scale; go.M = rows; go.N = D; go.K = D;
    if (b16) { go.C2 = base + L.hb; go.rss_out = (float*)(base + L.hss); }

    GemmArgs& g1 = ta.w1;  // g = GELU(W_1 RMS_mlp(h))
    g1.A = b16 ? (const void*)(base + L.hb) : (const void*)h; g1.lda = D; g1.W[0] = p.w1; g1.C[0] = g;
    g1.ldc = F; g1.seg_n = F; g1.eps = d->rms_eps; g1.M = rows; g1.N = F; g1.K = p.k1; g1.a_k = D;
    if (b16) { g1.rss_in = (const float*)(base + L.hss); g1.n_parts = parts; }

    GemmArgs& g2 = ta.w2;  // z = h + rho W_2 g
    g2.A = g; g2.lda = F; g2.W[0] = w->w_2; g2.C[0] = z; g2.ldc = D; g2.seg_n = D;
    g2.R = h; g2.ldr = D; g2.rscale = d->residual_scale; g2.M = rows; g2.N = D; g2.K = F;
    if (b16) g2.rss_out = (float*)(base + L.zss);

    if (kt) {
        GemmArgs& gk = ta.kv;  // persistent pair from the output z
        gk.A = z; gk.lda = D; gk.W[0] = p.wk; gk.W[1] = p.wv; gk.C[0] = kt; gk.C[1] = vt;
        gk.ldc = D; gk.seg_n = D; gk.eps = d->rms_eps; gk.M = rows; gk.N = 2 * D; gk.K = p.kq; gk.a_k = D;
        if (b16) { gk.rss_in = (const float*)(base + L.zss); gk.n_parts = parts; }
        if (!d->kv_source_norm) {  // the literal reading: W_k z_t, W_v z_t (the weights without g_attn)
            gk.W[0] = w->w_k; gk.W[1] = w->w_v; gk.K = D; gk.no_rms = 1;
        }
        if (d->flags & RT_FLAG_QK_NORM) { gk.qkn_mask = 1; gk.head_dim = d->attn.head_dim; gk.qkn_gain[0] = w->g_k; }
    }
    return ta;
}

// Everything after the attention, for `rows` rows (the products above, in order).
// fuse (bf16, head_dim 64): a blocked step of 1, 2 or 4 pairs ending at this
// position, run by the K/V projection's own workgroups once they have stored
// the pair (one launch fewer on the position's critical path).
rt_status enqueue_tail(const rt_layer_desc* d, const rt_layer_weights* w, const Projections& p, char* base,
                       const Layout& L, int64_t rows, const void* a, const void* x, void* z, void* kt, void* vt,
                       Launcher& run, const rt::UpdateArgs* fuse = nullptr) {
    using namespace rt;
    const rt_dtype dt = d->attn.dtype;
    hipStream_t s = run.s;
    TailArgs ta = tail_args(d, w, p, base, L, rows, a, x, z, kt, vt);
    RT_TRY(run.check(launch_gemm(dt, GemmKind::WO, ta.wo, s), "output projection"));
    RT_TRY(run.check(launch_gemm(dt, GemmKind::W1, ta.w1, s), "mlp up"));
    RT_TRY(run.check(launch_gemm(dt, GemmKind::W2, ta.w2, s), "mlp down"));
    if (!kt) return RT_OK;
    if (fuse) {
        ta.kv.upd = *fuse;
        return run.check(launch_gemm(dt, GemmKind::KV_UPDATE, ta.kv, s), "persistent kv projection + small step");
    }
    return run.check(launch_gemm(dt, GemmKind::KV, ta.kv, s), "persistent kv projection");
}

// The standard Transformer layer: the pairs come from the input, so every
// position is computed at once: one projection, one causal attention, and the
// tail over all N*B rows. The pairs are written straight into the caches.
rt_status enqueue_transformer(const rt_layer_desc* d, const rt_layer_weights* w, const void* x, void* z, void* kc,
                              void* vc, void* ws, Launcher& run) {
    using namespace rt;
    const int64_t rows = (int64_t)d->attn.seq_len * d->attn.batch;
    const Layout L = layout_of(d, Mode::Transformer);
    char* base = (char*)ws;
    Projections p;
    RT_TRY(enqueue_fold(d, w, base, L, run, &p));
    RT_TRY(enqueue_qkv(d, w, p, x, rows, base + L.q, kc, vc, (float*)(base + L.xss), run));
    UpdateArgs u{};
    u.q = base + L.q; u.k = kc; u.v = vc; u.a_out = base + L.a;
    u.P = (int64_t)d->attn.batch * d->attn.n_heads; u.nq = d->attn.seq_len;
    u.sigma2 = d->attn.softmax_scale * kLog2eHost; u.init = 1;
    RT_TRY(run.check(launch_causal_attention(d->attn.dtype, d->attn.head_dim, u, run.s), "causal attention"));
    return enqueue_tail(d, w, p, base, L, rows, base + L.a, x, z, nullptr, nullptr, run);
}

// Enqueue the whole layer forward on stream s (eager, or inside a capture).
rt_status enqueue_layer(const rt_layer_desc* d, const rt_layer_weights* w, const void* x, void* z, void* kc,
                        void* vc, void* ws, hipStream_t s, bool debug) {
    using namespace rt;
    Launcher run{s, debug};
    const Mode mode = mode_of(d);
    if (mode == Mode::Transformer) return enqueue_transformer(d, w, x, z, kc, vc, ws, run);

    const rt_dtype dt = d->attn.dtype;
    const size_t es = elem_bytes(dt);
    const int32_t N = d->attn.seq_len, B = d->attn.batch, H = d->attn.n_heads, dh = d->attn.head_dim;
    const Layout L = layout_of(d, mode);
    char* base = (char*)ws;
    void *q = base + L.q, *ke = base + L.ke, *ve = base + L.ve, *a = base + L.a;
    Projections p;
    RT_TRY(enqueue_fold(d, w, base, L, run, &p));

    // every query and ephemeral pair depends only on the input: one GEMM up front
    RT_TRY(enqueue_qkv(d, w, p, x, (int64_t)N * B, q, ke, ve, (float*)(base + L.xss), run));

    UpdateArgs u{};
    u.q = q; u.k = kc; u.v = vc; u.k_eph = ke; u.v_eph = ve; u.a_out = a;
    if (mode == Mode::Blocked) {
        u.m = (float*)(base + L.m); u.l = (float*)(base + L.l); u.o = (float*)(base + L.o);
    }
    u.P = (int64_t)B * H; u.sigma2 = d->attn.softmax_scale * kLog2eHost;
    // position 1: empty state, a_1 is its own ephemeral value
    u.kv0 = 0; u.nkv = 0; u.q0 = 0; u.nq = 1; u.init = 1; u.fin = 1;
    RT_TRY(run.check(launch_update(dt, dh, u, s), "finalize position 1"));

    const size_t slab = (size_t)B * d->d_model * es;
    // the blocked schedule's steps of 1, 2 and 4 pairs run inside the K/V projection (bf16, head_dim 64)
    // (not with at most 16 batch rows: the K/V product then runs on 16-row tiles, and the
    // fused form's one-head-per-tile layout would leave it a few workgroups)
    const bool fuse_small = mode == Mode::Blocked && dt == RT_BF16 && dh == 64 && B > 16;
    for (int32_t t = 1; t <= N; ++t) {
        const size_t at = (size_t)(t - 1) * slab;
        const int32_t bt = block_of(t);
        if (fuse_small && t < N && bt <= 4) {
            u.kv0 = t - bt; u.nkv = bt; u.q0 = t; u.nq = (bt < N - t) ? bt : N - t;
            u.init = (bt == t); u.fin = 1;
            RT_TRY(enqueue_tail(d, w, p, base, L, B, a, (const char*)x + at, (char*)z + at, (char*)kc + at,
                                (char*)vc + at, run, &u));
            continue;
        }
        RT_TRY(enqueue_tail(d, w, p, base, L, B, a, (const char*)x + at, (char*)z + at, (char*)kc + at,
                            (char*)vc + at, run));
        if (t == N) break;
        if (mode == Mode::Blocked) {
            // blocked step t, finishing query t+1 into a (its last merge)
            const int32_t b = block_of(t);
            u.kv0 = t - b; u.nkv = b; u.q0 = t; u.nq = (b < N - t) ? b : N - t;
            u.init = (b == t); u.fin = 1;
            RT_TRY(run.check(launch_update(dt, dh, u, s), "blocked update"));
        } else {
            // naive step: query t+1 reads every pair 1..t at once, then its ephemeral pair
            u.kv0 = 0; u.nkv = t; u.q0 = t; u.nq = 1; u.init = 1; u.fin = 1;
            RT_TRY(run.check(launch_update(dt, dh, u, s), "naive step"));
        }
    }
    return RT_OK;
}

// ---------------------------------------------------------------- stacks

// Positions whose queries and ephemeral pairs a stacked layer projects at once:
// a power of two, N/16 rounded down, at least 8.
int32_t stack_chunk(int32_t n) {
    int32_t c = 8;
    while ((int64_t)c * 2 * 16 <= n) c *= 2;
    return c;
}

// A stack of nl layers, layer l's input being layer l-1's output.
//
// Blocked layers run as a wavefront: at tick tau, layer l takes position
// t = tau - l*lag, and the per-position products of all layers at their
// positions share one launch each (one product at a time leaves most of the
// chip idle). Layer l >= 1 can only project a query once layer l-1 has made
// the position's input, so it projects its queries and ephemeral pairs in
// chunks of C positions, chunk [kC+1, (k+1)C] at position kC (lag = C + 8 >
// C keeps layer l-1 ahead of the chunk; a multiple of 8 keeps the blocks of
// 1, 2 and 4 pairs at the same ticks in every layer).
//
// The blocked schedule is kept exactly. Step t applies its block to queries
// t+1..t+b; those not yet projected (only when b > C, at t = kC: rows past
// t + C) get it when their chunk is projected, before any later step touches
// them (a step t' < (k+1)C reaches rows up to t' + lowbit(t') <= (k+1)C). Every query thus merges the same blocks in the same order as
// in the layer-by-layer run; a block of b > C pairs is read once per chunk of
// its deferred rows instead of once.
rt_status enqueue_stack(const rt_layer_desc* d, int32_t nl, const rt_layer_weights* w, const void* x,
                        void* const* z, void* const* kc, void* const* vc, void* ws, size_t stride, hipStream_t s,
                        bool debug) {
    using namespace rt;
    const Mode mode = mode_of(d);
    if (mode != Mode::Blocked || nl == 1) {  // layer after layer
        for (int32_t l = 0; l < nl; ++l)
            RT_TRY(enqueue_layer(d, &w[l], l ? z[l - 1] : x, z[l], kc[l], vc[l], (char*)ws + l * stride, s, debug));
        return RT_OK;
    }
    Launcher run{s, debug};
    const rt_dtype dt = d->attn.dtype;
    const size_t es = elem_bytes(dt);
    const int32_t N = d->attn.seq_len, B = d->attn.batch, H = d->attn.n_heads, dh = d->attn.head_dim;
    const Layout L = layout_of(d, mode);
    const size_t slab = (size_t)B * d->d_model * es;
    const int32_t C = stack_chunk(N), lag = C + 8;
    const bool fuse_small = dt == RT_BF16 && dh == 64 && B > 16;  // as in enqueue_layer

    struct Deferred {
        int32_t kv0, nkv, init;  // the block: key rows kv0..kv0+nkv-1 (0-based); its step initialises the rows
        int32_t r0, r1;          // query positions r0..r1 (1-based) still to receive it
    };
    struct Stacked {
        const rt_layer_weights* w;
        const char* x;
        char *z, *kc, *vc, *base;
        Projections p;
        UpdateArgs u;
        int32_t avail;                  // positions 1..avail have their queries and ephemeral pairs
        std::vector<Deferred> pending;  // in step order
    };
    std::vector<Stacked> ly(nl);
    for (int32_t l = 0; l < nl; ++l) {
        Stacked& y = ly[l];
        y.w = &w[l];
        y.x = (const char*)(l ? z[l - 1] : x);
        y.z = (char*)z[l];
        y.kc = (char*)kc[l];
        y.vc = (char*)vc[l];
        y.base = (char*)ws + l * stride;
        RT_TRY(enqueue_fold(d, y.w, y.base, L, run, &y.p));
        UpdateArgs& u = y.u;
        u = UpdateArgs{};
        u.q = y.base + L.q; u.k = y.kc; u.v = y.vc; u.k_eph = y.base + L.ke; u.v_eph = y.base + L.ve;
        u.a_out = y.base + L.a;
        u.m = (float*)(y.base + L.m); u.l = (float*)(y.base + L.l); u.o = (float*)(y.base + L.o);
        u.P = (int64_t)B * H; u.sigma2 = d->attn.softmax_scale * kLog2eHost;
        y.avail = 0;
    }
    auto update = [&](const Stacked& y, int32_t kv0, int32_t nkv, int32_t q0, int32_t nq, bool init, bool fin,
                      const char* what) {
        UpdateArgs u = y.u;
        u.kv0 = kv0; u.nkv = nkv; u.q0 = q0; u.nq = nq; u.init = init; u.fin = fin;
        return run.check(launch_update(dt, dh, u, s), what);
    };
    // queries and ephemeral pairs of positions avail+1..r1, then the deferred
    // blocks of those positions, oldest step first
    auto project = [&](Stacked& y, int32_t r1) -> rt_status {
        const int32_t r0 = y.avail + 1;
        const size_t at = (size_t)(r0 - 1) * slab;
        float* xss = (float*)(y.base + L.xss) + (size_t)(r0 - 1) * B * 4;
        RT_TRY(enqueue_qkv(d, y.w, y.p, y.x + at, (int64_t)(r1 - r0 + 1) * B, y.base + L.q + at,
                           y.base + L.ke + at, y.base + L.ve + at, xss, run));
        y.avail = r1;
        for (Deferred& e : y.pending) {
            const int32_t a = e.r0 > r0 ? e.r0 : r0, b = e.r1 < r1 ? e.r1 : r1;
            if (a > b) continue;
            RT_TRY(update(y, e.kv0, e.nkv, a - 1, b - a + 1, e.init != 0, false, "deferred blocked update"));
            e.r0 = b + 1;
        }
        size_t keep = 0;
        for (const Deferred& e : y.pending)
            if (e.r0 <= e.r1) y.pending[keep++] = e;
        y.pending.resize(keep);
        return RT_OK;
    };
    RT_TRY(project(ly[0], N));  // the first layer's input is given: every position up front

    std::vector<GemmArgs> go, g1, g2, gk, gku;
    std::vector<UpdateArgs> steps;
    std::vector<int32_t> act;
    const int64_t ticks = (int64_t)N + (int64_t)(nl - 1) * lag;
    for (int64_t tau = 1; tau <= ticks; ++tau) {
        act.clear();
        for (int32_t l = 0; l < nl; ++l) {
            const int64_t t = tau - (int64_t)l * lag;
            if (t >= 1 && t <= N) act.push_back(l);
        }
        go.clear(); g1.clear(); g2.clear(); gk.clear(); gku.clear();
        for (int32_t l : act) {
            Stacked& y = ly[l];
            const int32_t t = (int32_t)(tau - (int64_t)l * lag);
            // position t+1's query is read by this position's step: project its chunk
            // (layer l-1 has finished positions < t + lag, past the chunk's end)
            if (y.avail <= t && y.avail < N) {
                const int32_t r1 = (int64_t)y.avail + C < N ? y.avail + C : N;
                RT_TRY(project(y, r1));
            }
            if (t == 1)  // position 1: empty state, a_1 is its own ephemeral value
                RT_TRY(update(y, 0, 0, 0, 1, true, true, "finalize position 1"));
            const size_t at = (size_t)(t - 1) * slab;
            TailArgs ta = tail_args(d, y.w, y.p, y.base, L, B, y.base + L.a, y.x + at, y.z + at, y.kc + at,
                                    y.vc + at);
            go.push_back(ta.wo);
            g1.push_back(ta.w1);
            g2.push_back(ta.w2);
            const int32_t bt = block_of(t);
            if (fuse_small && t < N && bt <= 4) {
                UpdateArgs& u = ta.kv.upd;
                u = y.u;
                u.kv0 = t - bt; u.nkv = bt; u.q0 = t; u.nq = (bt < N - t) ? bt : N - t;
                u.init = (bt == t); u.fin = 1;
                gku.push_back(ta.kv);
            } else {
                gk.push_back(ta.kv);
            }
        }
        RT_TRY(run.check(launch_gemm_group(dt, GemmKind::WO, go.data(), (int)go.size(), s), "output projections"));
        RT_TRY(run.check(launch_gemm_group(dt, GemmKind::W1, g1.data(), (int)g1.size(), s), "mlp up"));
        RT_TRY(run.check(launch_gemm_group(dt, GemmKind::W2, g2.data(), (int)g2.size(), s), "mlp down"));
        if (gku.size() >= 2) {
            // several small steps: all the layers' pair projections in one launch
            // (larger tiles), then the steps in one launch (the fused form runs its
            // steps on the projection's 32-row tiles: 58.9 us per tick of six
            // layers, against 24.1 + the steps' own launch)
            steps.clear();
            for (GemmArgs& g : gku) {
                steps.push_back(g.upd);
                g.upd = UpdateArgs{};
                gk.push_back(g);
            }
            RT_TRY(run.check(launch_gemm_group(dt, GemmKind::KV, gk.data(), (int)gk.size(), s),
                             "persistent kv projections"));
            RT_TRY(run.check(launch_update_small_group(dt, dh, steps.data(), (int)steps.size(), s),
                             "small blocked steps"));
        } else {
            RT_TRY(run.check(launch_gemm_group(dt, GemmKind::KV_UPDATE, gku.data(), (int)gku.size(), s),
                             "persistent kv projection + small step"));
            RT_TRY(run.check(launch_gemm_group(dt, GemmKind::KV, gk.data(), (int)gk.size(), s),
                             "persistent kv projections"));
        }
        for (int32_t l : act) {
            Stacked& y = ly[l];
            const int32_t t = (int32_t)(tau - (int64_t)l * lag);
            const int32_t b = block_of(t);
            if (t == N || (fuse_small && b <= 4)) continue;
            // blocked step t: its block to queries t+1..t+b, finishing t+1; the
            // queries not yet projected get it when their chunk is
            const int32_t r1 = (int64_t)t + b < N ? t + b : N;
            const int32_t now = r1 < y.avail ? r1 : y.avail;
            RT_TRY(update(y, t - b, b, t, now - t, b == t, true, "blocked update"));
            if (r1 > now) y.pending.push_back(Deferred{t - b, b, b == t ? 1 : 0, now + 1, r1});
        }
    }
    for (const Stacked& y : ly)
        if (!y.pending.empty() || y.avail != N) return fail(RT_ERR_INTERNAL, "the stack schedule left work undone");
    return RT_OK;
}

// One position n_past+1 against caches holding the pairs of positions 1..n_past.
rt_status enqueue_decode(const rt_layer_desc* d, const rt_layer_weights* w, int32_t n_past, const void* x, void* z,
                         void* kc, void* vc, void* ws, hipStream_t s, bool debug) {
    using namespace rt;
    Launcher run{s, debug};
    const rt_dtype dt = d->attn.dtype;
    const int32_t B = d->attn.batch, H = d->attn.n_heads;
    const Layout L = layout_of(d, Mode::Decode);
    char* base = (char*)ws;
    const size_t at = (size_t)n_past * B * d->d_model * elem_bytes(dt);
    char *kt = (char*)kc + at, *vt = (char*)vc + at;
    const bool transformer = (d->flags & RT_FLAG_TRANSFORMER) != 0;
    Projections p;
    RT_TRY(enqueue_fold(d, w, base, L, run, &p));
    // a Transformer's pair of this position is its ephemeral pair: straight into the caches
    void* ke = transformer ? (void*)kt : (void*)(base + L.ke);
    void* ve = transformer ? (void*)vt : (void*)(base + L.ve);
    RT_TRY(enqueue_qkv(d, w, p, x, B, base + L.q, ke, ve, (float*)(base + L.xss), run));
    UpdateArgs u{};
    u.q = base + L.q; u.k = kc; u.v = vc; u.k_eph = ke; u.v_eph = ve; u.a_out = base + L.a;
    u.P = (int64_t)B * H; u.sigma2 = d->attn.softmax_scale * kLog2eHost;
    u.kv0 = 0; u.nkv = n_past; u.q0 = 0; u.nq = 1; u.init = 1; u.fin = 1;
    RT_TRY(run.check(launch_update(dt, d->attn.head_dim, u, s), "decode attention"));
    return enqueue_tail(d, w, p, base, L, B, base + L.a, x, z, transformer ? nullptr : kt,
                        transformer ? nullptr : vt, run);
}

// ---------------------------------------------------------------- backward

// The blocked attention of a whole sequence whose pairs are all known up front
// (u: q, k, v, k', v', m, l, o, lse, P and sigma2 set; a: [N][B][H][dh]
// outputs, slab bytes per position): position 1, then the schedule's levels
// from the largest block down, each level's steps in one launch. A query's
// blocks shrink from step to step, so it merges them in step order; each
// step's first query is finished by its level's launch, after its larger
// blocks.
rt_status enqueue_attention_levels(rt_dtype dt, int32_t dh, rt::UpdateArgs u, int32_t N, char* a, size_t slab,
                                   Launcher& run) {
    using namespace rt;
    u.a_out = a; u.kv0 = 0; u.nkv = 0; u.q0 = 0; u.nq = 1; u.init = 1; u.fin = 1; u.n_steps = 1;
    RT_TRY(run.check(launch_update(dt, dh, u, run.s), "finalize position 1"));
    int32_t top = 1;  // the largest power of two below N
    while ((int64_t)top * 2 < N) top *= 2;
    for (int32_t b = top; b >= 1 && b < N; b /= 2) {
        const int32_t steps = (N - 1 - b) / (2 * b) + 1;  // t = b, 3b, 5b, ... < N
        for (int32_t s0 = 0; s0 < steps; s0 += 65535) {
            const int32_t ns = steps - s0 < 65535 ? steps - s0 : 65535;
            const int32_t t = b + 2 * b * s0;  // this launch's first step
            u.kv0 = t - b; u.nkv = b; u.q0 = t; u.nq = (b < N - t) ? b : N - t;
            u.init = (t == b); u.fin = 1;
            u.a_out = a + (size_t)t * slab; u.a_step = (int64_t)(2 * (size_t)b * slab);
            u.n_steps = ns; u.n_pos = N;
            RT_TRY(run.check(launch_update(dt, dh, u, run.s), "blocked attention level"));
        }
    }
    return RT_OK;
}

rt_status check_backward(const rt_layer_desc* d) {
    RT_TRY(check_layer(d));
    if (d->flags & RT_FLAG_TRANSFORMER) return fail(RT_ERR_UNSUPPORTED, "the backward covers the RT layer only");
    if (d->flags & RT_FLAG_QK_NORM) return fail(RT_ERR_UNSUPPORTED, "the backward does not cover RT_FLAG_QK_NORM");
    if (!d->kv_source_norm) return fail(RT_ERR_UNSUPPORTED, "the backward covers kv_source_norm = 1 only");
    return RT_OK;
}

// Workspace of the layer backward (byte offsets, 256-aligned); NB = N*B rows.
struct BLayout {
    size_t wq, wk, wv, w1;                 // gain-folded weights (the recompute's products)
    size_t wkvT, w2T, w1T, woT, wqkvT;     // transposed weights (the adjoint products)
    size_t q, ke, ve, kc, vc, a;           // [NB][d] dtype: recomputed forward values
    size_t m, l, lse, delta;               // [N][P] fp32
    size_t o;                              // [NB][d] fp32: attention state, later the adjoint of RMS_attn(x)
    size_t h;                              // [NB][d] fp32
    size_t hb;                             // [NB][d] bf16 copy of h (bf16 layers)
    size_t hss;                            // [NB][d/32] fp32 partial sums of h^2 (bf16 layers)
    size_t u;                              // [NB][F] dtype: W_1 RMS(h), later GELU of it
    size_t kbar, vbar, qbar, kebar, vebar, abar, uzbar, mbar;  // [NB][d] fp32 adjoints
    size_t zbs, hbs;                       // [NB][d] dtype: rho * z_bar(total), rho * h_bar
    size_t ubar;                           // [NB][F] dtype
    size_t rz, rh, rx;                     // [NB] fp32: 1/rms of z, h, x
    size_t pkv;                            // [B][2d] dtype: k_bar|v_bar of one position
    size_t zt;                             // [B][d] fp32: z_bar(total) of one position
    size_t qkvb, kvb;                      // [NB][3d], [NB][2d] dtype: adjoints as product operands
    size_t gpart;                          // gain-gradient partial sums
    size_t xss;                            // [NB][4] fp32: quarter-row sums of x^2
    size_t wta, wtu, wpart;                // weight gradients: transposed operands and split partials
    int64_t wrows;                         // rows of the transposed operands (NB padded)
    size_t total;
};

BLayout blayout_of(const rt_layer_desc* d) {
    const size_t es = elem_bytes(d->attn.dtype);
    const size_t N = d->attn.seq_len, B = d->attn.batch, H = d->attn.n_heads, D = d->d_model, F = d->d_ff;
    const size_t NB = N * B, P = B * H;
    BLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    const size_t halves = d->attn.dtype == RT_BF16 ? 2 : 1;  // folded bf16 weights: two halves per row
    L.wq = take(halves * D * D * es); L.wk = take(halves * D * D * es); L.wv = take(halves * D * D * es);
    L.w1 = take(halves * F * D * es);
    L.wkvT = take(D * 2 * D * es); L.w2T = take(F * D * es); L.w1T = take(D * F * es); L.woT = take(D * D * es);
    L.wqkvT = take(D * 3 * D * es);
    L.q = take(NB * D * es); L.ke = take(NB * D * es); L.ve = take(NB * D * es);
    L.kc = take(NB * D * es); L.vc = take(NB * D * es); L.a = take(NB * D * es);
    L.m = take(N * P * 4); L.l = take(N * P * 4); L.lse = take(N * P * 4); L.delta = take(N * P * 4);
    L.o = take(NB * D * 4);
    L.h = take(NB * D * 4);
    L.hb = take(NB * D * 2);
    L.hss = take(D / rt::kRowSSTile * NB * 4 + 4);
    L.u = take(NB * F * es);
    L.kbar = take(NB * D * 4); L.vbar = take(NB * D * 4); L.qbar = take(NB * D * 4);
    L.kebar = take(NB * D * 4); L.vebar = take(NB * D * 4); L.abar = take(NB * D * 4);
    L.uzbar = take(NB * D * 4); L.mbar = take(NB * D * 4);
    L.zbs = take(NB * D * es); L.hbs = take(NB * D * es);
    L.ubar = take(NB * F * es);
    L.rz = take(NB * 4); L.rh = take(NB * 4); L.rx = take(NB * 4);
    L.pkv = take(B * 2 * D * es);
    L.zt = take(B * D * 4);
    L.qkvb = take(NB * 3 * D * es);
    L.kvb = take(NB * 2 * D * es);
    L.gpart = take((size_t)rt::gain_grad_blocks((int64_t)NB) * D * 4);
    L.xss = take(NB * 16);
    const rt::WgradPlan wp = rt::wgrad_plan((int64_t)NB);
    const size_t maxO = 3 * D > F ? 3 * D : F, maxI = D > F ? D : F;
    L.wrows = wp.rows_pad;
    L.wta = take(maxO * (size_t)wp.rows_pad * es);
    L.wtu = take(maxI * (size_t)wp.rows_pad * es);
    L.wpart = take((size_t)wp.splits * D * F * 4 > (size_t)wp.splits * 3 * D * D * 4 ? (size_t)wp.splits * D * F * 4
                                                                                      : (size_t)wp.splits * 3 * D * D * 4);
    L.total = off;
    return L;
}

rt_status enqueue_layer_backward(const rt_layer_desc* d, const rt_layer_weights* w, const void* x, const void* z,
                                 const float* z_bar, float* x_bar, const rt_layer_grads* gr, void* ws,
                                 hipStream_t s, bool debug) {
    using namespace rt;
    Launcher run{s, debug};
    const rt_dtype dt = d->attn.dtype;
    const bool b16 = dt == RT_BF16;
    const size_t es = elem_bytes(dt);
    const int32_t N = d->attn.seq_len, B = d->attn.batch, H = d->attn.n_heads, dh = d->attn.head_dim;
    const int32_t D = d->d_model, F = d->d_ff;
    const int64_t NB = (int64_t)N * B, P = (int64_t)B * H;
    const float rho = d->residual_scale, eps = d->rms_eps;
    const BLayout L = blayout_of(d);
    char* base = (char*)ws;
    auto at = [&](size_t off) { return (void*)(base + off); };
    auto f32 = [&](size_t off) { return (float*)(base + off); };

    // ---- weights: gain-folded for the recompute, transposed for the adjoint products
    Layout fl{};
    fl.wq = L.wq; fl.wk = L.wk; fl.wv = L.wv; fl.w1 = L.w1;
    Projections p;
    RT_TRY(enqueue_fold(d, w, base, fl, run, &p));
    RT_TRY(run.check(launch_transpose(dt, w->w_k, D, D, at(L.wkvT), 2 * D, 0, s), "transpose W_k"));
    RT_TRY(run.check(launch_transpose(dt, w->w_v, D, D, at(L.wkvT), 2 * D, D, s), "transpose W_v"));
    RT_TRY(run.check(launch_transpose(dt, w->w_2, D, F, at(L.w2T), D, 0, s), "transpose W_2"));
    RT_TRY(run.check(launch_transpose(dt, w->w_1, F, D, at(L.w1T), F, 0, s), "transpose W_1"));
    RT_TRY(run.check(launch_transpose(dt, w->w_o, D, D, at(L.woT), D, 0, s), "transpose W_o"));
    RT_TRY(run.check(launch_transpose(dt, w->w_q, D, D, at(L.wqkvT), 3 * D, 0, s), "transpose W_q"));
    RT_TRY(run.check(launch_transpose(dt, w->w_k, D, D, at(L.wqkvT), 3 * D, D, s), "transpose W_k"));
    RT_TRY(run.check(launch_transpose(dt, w->w_v, D, D, at(L.wqkvT), 3 * D, 2 * D, s), "transpose W_v"));

    // ---- recompute, batched over all N*B rows
    RT_TRY(enqueue_qkv(d, w, p, x, NB, at(L.q), at(L.ke), at(L.ve), f32(L.xss), run));
    {   // the persistent pairs from the stored outputs
        GemmArgs gk{};
        gk.A = z; gk.lda = D; gk.W[0] = p.wk; gk.W[1] = p.wv; gk.C[0] = at(L.kc); gk.C[1] = at(L.vc);
        gk.ldc = D; gk.seg_n = D; gk.eps = eps; gk.M = NB; gk.N = 2 * D; gk.K = p.kq; gk.a_k = D;
        RT_TRY(run.check(launch_gemm(dt, GemmKind::QKV, gk, s), "persistent pairs from z"));
    }
    {   // the blocked attention with each query's log-sum-exp (finishing query t+1 in step t)
        UpdateArgs u{};
        u.q = at(L.q); u.k = at(L.kc); u.v = at(L.vc); u.k_eph = at(L.ke); u.v_eph = at(L.ve);
        u.m = f32(L.m); u.l = f32(L.l); u.o = f32(L.o); u.lse = f32(L.lse); u.P = P;
        u.sigma2 = d->attn.softmax_scale * kLog2eHost;
        RT_TRY(enqueue_attention_levels(dt, dh, u, N, base + L.a, (size_t)B * D * es, run));
    }
    {   // h = x + rho W_o a (and, in bf16 layers, its bf16 copy and partial sums of h^2)
        GemmArgs go{};
        go.A = at(L.a); go.lda = D; go.W[0] = w->w_o; go.C[0] = f32(L.h); go.ldc = D; go.seg_n = D;
        go.R = x; go.ldr = D; go.rscale = rho; go.M = NB; go.N = D; go.K = D;
        if (b16) { go.C2 = at(L.hb); go.rss_out = f32(L.hss); }
        RT_TRY(run.check(launch_gemm(dt, GemmKind::WO, go, s), "h recompute"));
        GemmArgs g1{};  // u = W_1 RMS_mlp(h), before the GELU
        g1.A = b16 ? at(L.hb) : (const void*)f32(L.h); g1.lda = D; g1.W[0] = p.w1; g1.C[0] = at(L.u);
        g1.ldc = F; g1.seg_n = F; g1.eps = eps; g1.M = NB; g1.N = F; g1.K = p.k1; g1.a_k = D;
        if (b16) { g1.rss_in = f32(L.hss); g1.n_parts = D / kRowSSTile; }
        RT_TRY(run.check(launch_gemm(dt, GemmKind::W1_PRE, g1, s), "u recompute"));
    }

    // ---- positions in reverse
    RT_TRY(run.check(launch_zero_f32(f32(L.kbar), NB * D, s), "clear k_bar"));
    RT_TRY(run.check(launch_zero_f32(f32(L.vbar), NB * D, s), "clear v_bar"));
    BackwardArgs bw{};
    bw.q = at(L.q); bw.k_eph = at(L.ke); bw.v_eph = at(L.ve); bw.k = at(L.kc); bw.v = at(L.vc); bw.a = at(L.a);
    bw.lse = f32(L.lse); bw.a_bar = f32(L.abar); bw.q_bar = f32(L.qbar); bw.k_eph_bar = f32(L.kebar);
    bw.v_eph_bar = f32(L.vebar); bw.k_bar = f32(L.kbar); bw.v_bar = f32(L.vbar); bw.delta = f32(L.delta);
    bw.P = P; bw.n_pos = N; bw.sigma = d->attn.softmax_scale; bw.sigma2 = d->attn.softmax_scale * kLog2eHost;
    bw.kv_accumulate = 1;
    auto plain = [&](const void* A, int64_t lda, const void* W, int n, int k, float* C, const char* what) {
        GemmArgs g{};
        g.A = A; g.lda = lda; g.W[0] = W; g.C[0] = C; g.ldc = n; g.seg_n = n; g.M = B; g.N = n; g.K = k;
        return run.check(launch_gemm(dt, GemmKind::PLAIN, g, s), what);
    };
    const size_t rowsD = (size_t)B * D, rowsF = (size_t)B * F;
    for (int32_t j = N - 1; j >= 0; --j) {
        if (j + 1 < N) {  // step t = j + 1: keys (t-b, t] against queries (t, t+b]
            const int32_t t = j + 1, b = block_of(t);
            RT_TRY(run.check(launch_backward_step(dt, dh, bw, t - b, b, t, (b < N - t) ? b : N - t, s),
                             "attention rectangle"));
        }
        float* kb = f32(L.kbar) + j * rowsD;
        float* vb = f32(L.vbar) + j * rowsD;
        float* uzb = f32(L.uzbar) + j * rowsD;
        RT_TRY(run.check(launch_pack(dt, at(L.pkv), 2 * D, kb, vb, nullptr, 2, B, D, 1.f, s), "pack k_bar|v_bar"));
        RT_TRY(plain(at(L.pkv), 2 * D, at(L.wkvT), D, 2 * D, uzb, "W_kv^T product"));
        void* zbs = base + L.zbs + j * rowsD * es;
        RT_TRY(run.check(launch_rms_bwd(dt, dt, (const char*)z + j * rowsD * es, uzb, w->g_attn, eps,
                                        z_bar + j * rowsD, f32(L.zt), zbs, rho, f32(L.rz) + (int64_t)j * B, B, D, s),
                         "RMS_attn adjoint of z"));
        void* ub = base + L.ubar + j * rowsF * es;
        {   // u_bar = (W_2^T rho z_bar) * GELU'(u_j)
            GemmArgs g2{};
            g2.A = zbs; g2.lda = D; g2.W[0] = at(L.w2T); g2.C[0] = ub; g2.ldc = F; g2.seg_n = F;
            g2.R = base + L.u + j * rowsF * es; g2.ldr = F; g2.M = B; g2.N = F; g2.K = D;
            RT_TRY(run.check(launch_gemm(dt, GemmKind::W2_BWD, g2, s), "W_2^T product and GELU adjoint"));
        }
        float* mb = f32(L.mbar) + j * rowsD;
        RT_TRY(plain(ub, F, at(L.w1T), D, F, mb, "W_1^T product"));
        void* hbs = base + L.hbs + j * rowsD * es;
        RT_TRY(run.check(launch_rms_bwd(RT_F32, dt, f32(L.h) + j * rowsD, mb, w->g_mlp, eps, f32(L.zt),
                                        x_bar + j * rowsD, hbs, rho, f32(L.rh) + (int64_t)j * B, B, D, s),
                         "RMS_mlp adjoint of h"));
        RT_TRY(plain(hbs, D, at(L.woT), D, D, f32(L.abar) + j * rowsD, "W_o^T product"));
        {   // query j's own pass: D_j, the ephemeral pair's gradients, q_bar's first term
            BackwardArgs bj = bw;
            const size_t eo = (size_t)j * rowsD * es;
            bj.q = base + L.q + eo; bj.k_eph = base + L.ke + eo; bj.v_eph = base + L.ve + eo; bj.a = base + L.a + eo;
            bj.lse = f32(L.lse) + (int64_t)j * P; bj.delta = f32(L.delta) + (int64_t)j * P;
            bj.a_bar = f32(L.abar) + j * rowsD; bj.q_bar = f32(L.qbar) + j * rowsD;
            bj.k_eph_bar = f32(L.kebar) + j * rowsD; bj.v_eph_bar = f32(L.vebar) + j * rowsD;
            bj.n_pos = 1;
            RT_TRY(run.check(launch_backward_prep(dt, dh, bj, s), "query pass"));
        }
    }

    // ---- batched: the input's adjoint through RMS_attn(x)
    float* uxb = f32(L.o);  // (the attention state is no longer needed)
    RT_TRY(run.check(launch_pack(dt, at(L.qkvb), 3 * D, f32(L.qbar), f32(L.kebar), f32(L.vebar), 3, NB, D, 1.f, s),
                     "pack q_bar|k'_bar|v'_bar"));
    {
        GemmArgs g{};
        g.A = at(L.qkvb); g.lda = 3 * D; g.W[0] = at(L.wqkvT); g.C[0] = uxb; g.ldc = D; g.seg_n = D;
        g.M = NB; g.N = D; g.K = 3 * D;
        RT_TRY(run.check(launch_gemm(dt, GemmKind::PLAIN, g, s), "W_qkv^T product"));
    }
    RT_TRY(run.check(launch_rms_bwd(dt, dt, x, uxb, w->g_attn, eps, x_bar, x_bar, nullptr, 1.f, f32(L.rx), NB, D, s),
                     "RMS_attn adjoint of x"));

    // ---- weight gradients: the products' inputs, materialised (q, k', v' are no longer needed)
    void* ux = at(L.q);
    void* uz = at(L.ke);
    void* mm = at(L.ve);
    RT_TRY(run.check(launch_rms_apply(dt, dt, x, w->g_attn, eps, ux, NB, D, s), "RMS_attn(x)"));
    RT_TRY(run.check(launch_rms_apply(dt, dt, z, w->g_attn, eps, uz, NB, D, s), "RMS_attn(z)"));
    RT_TRY(run.check(launch_rms_apply(RT_F32, dt, f32(L.h), w->g_mlp, eps, mm, NB, D, s), "RMS_mlp(h)"));
    RT_TRY(run.check(launch_pack(dt, at(L.kvb), 2 * D, f32(L.kbar), f32(L.vbar), nullptr, 2, NB, D, 1.f, s),
                     "pack k_bar|v_bar"));
    RT_TRY(run.check(launch_gelu_inplace(dt, at(L.u), NB * F, s), "GELU(u)"));
    const char* qkvb = base + L.qkvb;
    const char* kvb = base + L.kvb;
    // each a sum over all N*B rows of (adjoint of the product's output)^T (its input); the
    // products sharing an input follow each other, which transposes that input once
    const WgradScratch wsc{at(L.wta), at(L.wtu), f32(L.wpart), L.wrows};
    auto wgrad = [&](const void* abar, int64_t lda, const void* u, int64_t ldu, int O, int I, float* out, bool acc,
                     bool u_ready, const char* what) {
        return run.check(weight_grad(dt, abar, lda, u, ldu, NB, O, I, out, acc, u_ready, wsc, s), what);
    };
    RT_TRY(wgrad(qkvb, 3 * D, ux, D, D, D, gr->w_q, false, false, "W_q gradient"));
    RT_TRY(wgrad(qkvb + D * es, 3 * D, ux, D, D, D, gr->w_k, false, true, "W_k gradient"));
    RT_TRY(wgrad(qkvb + 2 * D * es, 3 * D, ux, D, D, D, gr->w_v, false, true, "W_v gradient"));
    RT_TRY(wgrad(kvb, 2 * D, uz, D, D, D, gr->w_k, true, false, "W_k gradient"));
    RT_TRY(wgrad(kvb + D * es, 2 * D, uz, D, D, D, gr->w_v, true, true, "W_v gradient"));
    RT_TRY(wgrad(at(L.hbs), D, at(L.a), D, D, D, gr->w_o, false, false, "W_o gradient"));
    RT_TRY(wgrad(at(L.ubar), F, mm, D, F, D, gr->w_1, false, false, "W_1 gradient"));
    RT_TRY(wgrad(at(L.zbs), D, at(L.u), F, D, F, gr->w_2, false, false, "W_2 gradient"));
    if (gr->g_attn) {
        RT_TRY(run.check(launch_gain_grad(dt, uxb, x, f32(L.rx), NB, D, f32(L.gpart), gr->g_attn, 0, s), "g_attn"));
        RT_TRY(run.check(launch_gain_grad(dt, f32(L.uzbar), z, f32(L.rz), NB, D, f32(L.gpart), gr->g_attn, 1, s),
                         "g_attn"));
    }
    if (gr->g_mlp)
        RT_TRY(run.check(launch_gain_grad(RT_F32, f32(L.mbar), f32(L.h), f32(L.rh), NB, D, f32(L.gpart), gr->g_mlp,
                                          0, s),
                         "g_mlp"));
    return RT_OK;
}

}  // namespace

struct rt_plan {
    std::vector<hipGraph_t> graphs;    // replayed in order
    std::vector<hipGraphExec_t> execs;
};

namespace {

constexpr int32_t kMaxStackLayers = 1024;

rt_status check_stack(const rt_layer_desc* d, int32_t nl, const rt_layer_weights* w, const void* x, void* const* z,
                      void* const* kc, void* const* vc, void* ws, size_t ws_bytes) {
    RT_TRY(check_layer(d));
    if (nl < 1 || nl > kMaxStackLayers)
        return fail(RT_ERR_INVALID_ARG, "n_layers=%d outside 1..%d", nl, kMaxStackLayers);
    if (!w || !z || !kc || !vc) return fail(RT_ERR_INVALID_ARG, "weights, z, k_cache or v_cache array is NULL");
    for (int32_t l = 0; l < nl; ++l) {
        const rt_status st = check_layer_ptrs(&w[l], l ? z[l - 1] : x, z[l], kc[l], vc[l], ws);
        if (st != RT_OK) return fail(st, "layer %d: %s", l, g_last_error.c_str());
    }
    const size_t need = (size_t)nl * layout_of(d, mode_of(d)).total;
    if (ws_bytes < need) return fail(RT_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, need);
    return RT_OK;
}

// Capture what enqueue puts on a stream into HIP graphs (see CaptureSegments), instantiated.
template <typename F>
rt_status capture_plan(F&& enqueue, rt_plan** plan) {
    hipStream_t cs;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e, "capture stream");
    rt_plan* p = new rt_plan();
    auto drop = [&](rt_status st) {
        for (hipGraphExec_t x : p->execs) (void)hipGraphExecDestroy(x);
        for (hipGraph_t g : p->graphs) (void)hipGraphDestroy(g);
        delete p;
        return st;
    };
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return drop(hip_fail(e, "hipStreamBeginCapture"));
    }
    CaptureSegments seg;
    seg.s = cs;
    g_capture = &seg;
    rt_status st = enqueue(cs);
    g_capture = nullptr;
    hipGraph_t last = nullptr;
    e = hipStreamEndCapture(cs, &last);
    (void)hipStreamDestroy(cs);
    p->graphs = std::move(seg.graphs);
    if (last) {
        size_t nodes = 0;  // a capture cut right after the last launch leaves an empty graph
        if (hipGraphGetNodes(last, nullptr, &nodes) == hipSuccess && nodes == 0 && !p->graphs.empty())
            (void)hipGraphDestroy(last);
        else
            p->graphs.push_back(last);
    }
    if (st != RT_OK) return drop(st);
    if (e != hipSuccess) return drop(hip_fail(e, "hipStreamEndCapture"));
    for (hipGraph_t g : p->graphs) {
        hipGraphExec_t x = nullptr;
        e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
        if (e != hipSuccess) return drop(hip_fail(e, "hipGraphInstantiate"));
        p->execs.push_back(x);
    }
    *plan = p;
    return RT_OK;
}

}  // namespace

namespace rt {

rt_status set_error(rt_status st, const char* a, const char* b) { return fail(st, "%s%s", a, b); }

rt_status check_decode_args(const rt_layer_desc* desc, const rt_layer_weights* w, int32_t n_past, const void* x_t,
                            void* z_t, void* k_cache, void* v_cache) {
    RT_TRY(check_layer(desc));
    // (the workspace is checked by the caller; a stand-in aligned address here)
    RT_TRY(check_layer_ptrs(w, x_t, z_t, k_cache, v_cache, reinterpret_cast<void*>(uintptr_t(256))));
    if (n_past < 0 || n_past >= desc->attn.seq_len)
        return fail(RT_ERR_INVALID_ARG, "n_past=%d outside 0..%d (seq_len is the cache capacity)", n_past,
                    desc->attn.seq_len - 1);
    return RT_OK;
}

}  // namespace rt

extern "C" {

const char* rt_last_error(void) { return g_last_error.c_str(); }

rt_status rt_schedule_step(int32_t t, int32_t n, int32_t* kv_first, int32_t* kv_last, int32_t* q_first,
                           int32_t* q_last) {
    if (!kv_first || !kv_last || !q_first || !q_last) return fail(RT_ERR_INVALID_ARG, "output pointer is NULL");
    if (n <= 0 || t < 1 || t > n) return fail(RT_ERR_INVALID_ARG, "need 1 <= t <= n (t=%d, n=%d)", t, n);
    const int32_t b = block_of(t);
    *kv_first = t - b + 1;
    *kv_last = t;
    *q_first = t + 1;
    *q_last = (int64_t)t + b < (int64_t)n ? t + b : n;
    return RT_OK;
}

rt_status rt_blocked_attn_update(const rt_attn_desc* desc, int32_t t, const void* q, const void* k, const void* v,
                                 float* m, float* l, float* o, rt_stream_t stream) {
    RT_TRY(check_attn(desc));
    if (t < 1 || t > desc->seq_len) return fail(RT_ERR_INVALID_ARG, "t=%d outside 1..%d", t, desc->seq_len);
    const void* ps[] = {q, k, v, m, l, o};
    const char* names[] = {"q", "k", "v", "m", "l", "o"};
    for (int i = 0; i < 6; ++i) {
        if (!ps[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned16(ps[i]) && i != 3 && i != 4) return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (((uintptr_t)m & 3u) || ((uintptr_t)l & 3u)) return fail(RT_ERR_INVALID_ARG, "m and l must be 4-byte aligned");
    const int32_t N = desc->seq_len, b = block_of(t);
    const int32_t nq = (b < N - t) ? b : N - t;
    if (nq <= 0) return RT_OK;
    rt::UpdateArgs u{};
    u.q = q; u.k = k; u.v = v; u.m = m; u.l = l; u.o = o;
    u.P = (int64_t)desc->batch * desc->n_heads;
    u.kv0 = t - b; u.nkv = b; u.q0 = t; u.nq = nq;
    u.sigma2 = desc->softmax_scale * rt::kLog2eHost;
    u.init = (b == t); u.fin = 0;
    hipError_t e = rt::launch_update(desc->dtype, desc->head_dim, u, (hipStream_t)stream);
    return e == hipSuccess ? RT_OK : hip_fail(e, "rt_blocked_attn_update launch");
}

rt_status rt_finalize_step(const rt_attn_desc* desc, int32_t t, const void* q, const void* k_eph,
                           const void* v_eph, const float* m, const float* l, const float* o, void* a_t,
                           rt_stream_t stream) {
    RT_TRY(check_attn(desc));
    if (t < 1 || t > desc->seq_len) return fail(RT_ERR_INVALID_ARG, "t=%d outside 1..%d", t, desc->seq_len);
    const void* ps[] = {q, k_eph, v_eph, a_t};
    const char* names[] = {"q", "k_eph", "v_eph", "a_t"};
    for (int i = 0; i < 4; ++i) {
        if (!ps[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned16(ps[i])) return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (t > 1) {
        if (!m || !l || !o) return fail(RT_ERR_INVALID_ARG, "state is NULL");
        if (!aligned16(o) || ((uintptr_t)m & 3u) || ((uintptr_t)l & 3u))
            return fail(RT_ERR_INVALID_ARG, "state is misaligned");
    }
    rt::UpdateArgs u{};
    u.q = q; u.k_eph = k_eph; u.v_eph = v_eph;
    u.m = const_cast<float*>(m); u.l = const_cast<float*>(l); u.o = const_cast<float*>(o);
    u.a_out = a_t;
    u.P = (int64_t)desc->batch * desc->n_heads;
    u.kv0 = 0; u.nkv = 0; u.q0 = t - 1; u.nq = 1;
    u.sigma2 = desc->softmax_scale * rt::kLog2eHost;
    u.init = (t == 1); u.fin = 1;
    hipError_t e = rt::launch_update(desc->dtype, desc->head_dim, u, (hipStream_t)stream);
    return e == hipSuccess ? RT_OK : hip_fail(e, "rt_finalize_step launch");
}

rt_status rt_update_finalize_step(const rt_attn_desc* desc, int32_t t, const void* q, const void* k_eph,
                                  const void* v_eph, const void* k, const void* v, float* m, float* l, float* o,
                                  void* a_next, rt_stream_t stream) {
    RT_TRY(check_attn(desc));
    if (t < 1 || t >= desc->seq_len) return fail(RT_ERR_INVALID_ARG, "t=%d outside 1..%d", t, desc->seq_len - 1);
    const void* ps[] = {q, k_eph, v_eph, k, v, m, l, o, a_next};
    const char* names[] = {"q", "k_eph", "v_eph", "k", "v", "m", "l", "o", "a_next"};
    for (int i = 0; i < 9; ++i) {
        if (!ps[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned16(ps[i]) && i != 5 && i != 6) return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (((uintptr_t)m & 3u) || ((uintptr_t)l & 3u)) return fail(RT_ERR_INVALID_ARG, "m and l must be 4-byte aligned");
    const int32_t N = desc->seq_len, b = block_of(t);
    rt::UpdateArgs u{};
    u.q = q; u.k = k; u.v = v; u.k_eph = k_eph; u.v_eph = v_eph; u.m = m; u.l = l; u.o = o; u.a_out = a_next;
    u.P = (int64_t)desc->batch * desc->n_heads;
    u.kv0 = t - b; u.nkv = b; u.q0 = t; u.nq = (b < N - t) ? b : N - t;
    u.sigma2 = desc->softmax_scale * rt::kLog2eHost;
    u.init = (b == t); u.fin = 1;
    hipError_t e = rt::launch_update(desc->dtype, desc->head_dim, u, (hipStream_t)stream);
    return e == hipSuccess ? RT_OK : hip_fail(e, "rt_update_finalize_step launch");
}

rt_status rt_attn_forward(const rt_attn_desc* desc, const void* q, const void* k_eph, const void* v_eph,
                          const void* k, const void* v, void* a, float* lse, float* m, float* l, float* o,
                          rt_stream_t stream) {
    RT_TRY(check_attn(desc));
    const void* ps[] = {q, k_eph, v_eph, k, v, a, lse, m, l, o};
    const char* names[] = {"q", "k_eph", "v_eph", "k", "v", "a", "lse", "m", "l", "o"};
    for (int i = 0; i < 10; ++i) {
        if (!ps[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned16(ps[i]) && i != 6 && i != 7 && i != 8)
            return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (((uintptr_t)lse & 3u) || ((uintptr_t)m & 3u) || ((uintptr_t)l & 3u))
        return fail(RT_ERR_INVALID_ARG, "lse, m and l must be 4-byte aligned");
    const int32_t N = desc->seq_len;
    const size_t slab = (size_t)desc->batch * desc->n_heads * desc->head_dim * elem_bytes(desc->dtype);
    rt::UpdateArgs u{};
    u.q = q; u.k = k; u.v = v; u.k_eph = k_eph; u.v_eph = v_eph; u.m = m; u.l = l; u.o = o; u.lse = lse;
    u.P = (int64_t)desc->batch * desc->n_heads;
    u.sigma2 = desc->softmax_scale * rt::kLog2eHost;
    Launcher run{(hipStream_t)stream, false};
    return enqueue_attention_levels(desc->dtype, desc->head_dim, u, N, (char*)a, slab, run);
}

rt_status rt_attn_backward(const rt_attn_desc* desc, const void* q, const void* k_eph, const void* v_eph,
                           const void* k, const void* v, const void* a, const float* lse, const float* a_bar,
                           float* q_bar, float* k_eph_bar, float* v_eph_bar, float* k_bar, float* v_bar,
                           float* delta, rt_stream_t stream) {
    RT_TRY(check_attn(desc));
    const void* ps[] = {q, k_eph, v_eph, k, v, a, lse, a_bar, q_bar, k_eph_bar, v_eph_bar, k_bar, v_bar, delta};
    const char* names[] = {"q", "k_eph", "v_eph", "k", "v", "a", "lse", "a_bar", "q_bar", "k_eph_bar",
                           "v_eph_bar", "k_bar", "v_bar", "delta"};
    for (int i = 0; i < 14; ++i) {
        if (!ps[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", names[i]);
        if (!aligned16(ps[i]) && i != 6 && i != 13)
            return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (((uintptr_t)lse & 3u) || ((uintptr_t)delta & 3u))
        return fail(RT_ERR_INVALID_ARG, "lse and delta must be 4-byte aligned");
    const int32_t N = desc->seq_len, dh = desc->head_dim;
    hipStream_t s = (hipStream_t)stream;
    rt::BackwardArgs bw{};
    bw.q = q; bw.k_eph = k_eph; bw.v_eph = v_eph; bw.k = k; bw.v = v; bw.a = a; bw.lse = lse; bw.a_bar = a_bar;
    bw.q_bar = q_bar; bw.k_eph_bar = k_eph_bar; bw.v_eph_bar = v_eph_bar; bw.k_bar = k_bar; bw.v_bar = v_bar;
    bw.delta = delta; bw.P = (int64_t)desc->batch * desc->n_heads; bw.n_pos = N;
    bw.sigma = desc->softmax_scale; bw.sigma2 = desc->softmax_scale * rt::kLog2eHost;
    hipError_t e = rt::launch_backward_prep(desc->dtype, dh, bw, s);
    // the forward's steps in order: step t's rectangle sets key row t (its first visit)
    for (int32_t t = 1; t < N && e == hipSuccess; ++t) {
        const int32_t b = block_of(t);
        e = rt::launch_backward_step(desc->dtype, dh, bw, t - b, b, t, (b < N - t) ? b : N - t, s);
    }
    // the last position's pair is read by no query
    if (e == hipSuccess) e = rt::launch_backward_zero_rows(dh, bw, N - 1, 1, s);
    return e == hipSuccess ? RT_OK : hip_fail(e, "rt_attn_backward launch");
}

size_t rt_layer_workspace_bytes(const rt_layer_desc* desc) {
    if (check_layer(desc) != RT_OK) return 0;
    return layout_of(desc, mode_of(desc)).total;
}

size_t rt_layer_backward_workspace_bytes(const rt_layer_desc* desc) {
    if (check_backward(desc) != RT_OK) return 0;
    return blayout_of(desc).total;
}

rt_status rt_layer_backward(const rt_layer_desc* desc, const rt_layer_weights* w, const void* x, const void* z,
                            const float* z_bar, float* x_bar, const rt_layer_grads* grads, void* workspace,
                            size_t workspace_bytes, rt_stream_t stream) {
    RT_TRY(check_backward(desc));
    if (!w) return fail(RT_ERR_INVALID_ARG, "weights is NULL");
    {
        const void* ps[] = {w->w_q, w->w_k, w->w_v, w->w_o, w->w_1, w->w_2, x, z, z_bar, x_bar, workspace};
        const char* names[] = {"w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "x", "z", "z_bar", "x_bar", "workspace"};
        for (int i = 0; i < 11; ++i) {
            if (!ps[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", names[i]);
            if (!aligned16(ps[i])) return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
        }
        if (((uintptr_t)workspace & 255u) != 0) return fail(RT_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
        if ((w->g_attn && !aligned16(w->g_attn)) || (w->g_mlp && !aligned16(w->g_mlp)))
            return fail(RT_ERR_INVALID_ARG, "gains must be 16-byte aligned");
    }
    if (!grads) return fail(RT_ERR_INVALID_ARG, "grads is NULL");
    const float* gp[] = {grads->w_q, grads->w_k, grads->w_v, grads->w_o, grads->w_1, grads->w_2};
    const char* gn[] = {"grads->w_q", "grads->w_k", "grads->w_v", "grads->w_o", "grads->w_1", "grads->w_2"};
    for (int i = 0; i < 6; ++i) {
        if (!gp[i]) return fail(RT_ERR_INVALID_ARG, "%s is NULL", gn[i]);
        if (!aligned16(gp[i])) return fail(RT_ERR_INVALID_ARG, "%s is not 16-byte aligned", gn[i]);
    }
    if ((grads->g_attn && ((uintptr_t)grads->g_attn & 3u)) || (grads->g_mlp && ((uintptr_t)grads->g_mlp & 3u)))
        return fail(RT_ERR_INVALID_ARG, "gain gradients must be 4-byte aligned");
    const size_t need = blayout_of(desc).total;
    if (workspace_bytes < need)
        return fail(RT_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return enqueue_layer_backward(desc, w, x, z, z_bar, x_bar, grads, workspace, (hipStream_t)stream,
                                  (desc->flags & RT_FLAG_DEBUG_SYNC) != 0);
}

size_t rt_layer_decode_workspace_bytes(const rt_layer_desc* desc) {
    if (check_layer(desc) != RT_OK) return 0;
    return layout_of(desc, Mode::Decode).total;
}

rt_status rt_layer_decode_step(const rt_layer_desc* desc, const rt_layer_weights* w, int32_t n_past,
                               const void* x_t, void* z_t, void* k_cache, void* v_cache, void* workspace,
                               size_t workspace_bytes, rt_stream_t stream) {
    RT_TRY(rt::check_decode_args(desc, w, n_past, x_t, z_t, k_cache, v_cache));
    RT_TRY(check_layer_ptrs(w, x_t, z_t, k_cache, v_cache, workspace));
    const size_t need = layout_of(desc, Mode::Decode).total;
    if (workspace_bytes < need)
        return fail(RT_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return enqueue_decode(desc, w, n_past, x_t, z_t, k_cache, v_cache, workspace, (hipStream_t)stream,
                          (desc->flags & RT_FLAG_DEBUG_SYNC) != 0);
}

rt_status rt_layer_forward(const rt_layer_desc* desc, const rt_layer_weights* w, const void* x, void* z,
                           void* k_cache, void* v_cache, void* workspace, size_t workspace_bytes,
                           rt_stream_t stream) {
    RT_TRY(check_layer(desc));
    RT_TRY(check_layer_ptrs(w, x, z, k_cache, v_cache, workspace));
    const size_t need = layout_of(desc, mode_of(desc)).total;
    if (workspace_bytes < need)
        return fail(RT_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return enqueue_layer(desc, w, x, z, k_cache, v_cache, workspace, (hipStream_t)stream,
                         (desc->flags & RT_FLAG_DEBUG_SYNC) != 0);
}

rt_status rt_layer_plan_create(const rt_layer_desc* desc, const rt_layer_weights* w, const void* x, void* z,
                               void* k_cache, void* v_cache, void* workspace, size_t workspace_bytes,
                               rt_plan** plan) {
    if (!plan) return fail(RT_ERR_INVALID_ARG, "plan is NULL");
    *plan = nullptr;
    RT_TRY(check_layer(desc));
    RT_TRY(check_layer_ptrs(w, x, z, k_cache, v_cache, workspace));
    const size_t need = layout_of(desc, mode_of(desc)).total;
    if (workspace_bytes < need)
        return fail(RT_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    return capture_plan([&](hipStream_t cs) { return enqueue_layer(desc, w, x, z, k_cache, v_cache, workspace, cs, false); },
                        plan);
}

size_t rt_stack_workspace_bytes(const rt_layer_desc* desc, int32_t n_layers) {
    if (check_layer(desc) != RT_OK || n_layers < 1 || n_layers > kMaxStackLayers) return 0;
    return (size_t)n_layers * layout_of(desc, mode_of(desc)).total;
}

rt_status rt_stack_forward(const rt_layer_desc* desc, int32_t n_layers, const rt_layer_weights* w, const void* x,
                           void* const* z, void* const* k_cache, void* const* v_cache, void* workspace,
                           size_t workspace_bytes, rt_stream_t stream) {
    RT_TRY(check_stack(desc, n_layers, w, x, z, k_cache, v_cache, workspace, workspace_bytes));
    return enqueue_stack(desc, n_layers, w, x, z, k_cache, v_cache, workspace, layout_of(desc, mode_of(desc)).total,
                         (hipStream_t)stream, (desc->flags & RT_FLAG_DEBUG_SYNC) != 0);
}

rt_status rt_stack_plan_create(const rt_layer_desc* desc, int32_t n_layers, const rt_layer_weights* w, const void* x,
                               void* const* z, void* const* k_cache, void* const* v_cache, void* workspace,
                               size_t workspace_bytes, rt_plan** plan) {
    if (!plan) return fail(RT_ERR_INVALID_ARG, "plan is NULL");
    *plan = nullptr;
    RT_TRY(check_stack(desc, n_layers, w, x, z, k_cache, v_cache, workspace, workspace_bytes));
    const size_t stride = layout_of(desc, mode_of(desc)).total;
    return capture_plan(
        [&](hipStream_t cs) {
            return enqueue_stack(desc, n_layers, w, x, z, k_cache, v_cache, workspace, stride, cs, false);
        },
        plan);
}

rt_status rt_layer_plan_launch(rt_plan* plan, rt_stream_t stream) {
    if (!plan || plan->execs.empty()) return fail(RT_ERR_INVALID_ARG, "plan is NULL");
    for (hipGraphExec_t x : plan->execs) {
        hipError_t e = hipGraphLaunch(x, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    }
    return RT_OK;
}

void rt_layer_plan_destroy(rt_plan* plan) {
    if (!plan) return;
    for (hipGraphExec_t x : plan->execs) (void)hipGraphExecDestroy(x);
    for (hipGraph_t g : plan->graphs) (void)hipGraphDestroy(g);
    delete plan;
}

}  // extern "C"
