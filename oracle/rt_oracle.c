/*
 * CPU oracle for the Recurrent Transformer (RT) layer -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct implementation of what the GPU library
 * computes, used by the tests, the smoke check and the bench's CPU baseline
 * to judge it. The GPU library never links, loads or calls this file, and
 * this file uses nothing from the library.
 *
 * It follows the definitions on the Recurrent Transformer reading note
 * (lshu.cn/news/403416):
 *   - translated paper, section 2 "Notation": the attention operator
 *     Attn((k_1,v_1)..(k_l,v_l), q) = sum_i v_i exp<k_i,q> / sum_j exp<k_j,q>,
 *     RMS normalisation, pre-LN residual branches, per-head construction
 *     followed by the usual output projection;
 *   - translated paper, section 2.1: queries, keys and values of a position
 *     come from Q/K/V applied to RMS(x_i); the layer output adds the
 *     attention branch and then the MLP branch to the input;
 *   - translated paper, section 2.2, and summary section 2.2: the RT layer
 *     forms an ephemeral key/value pair from the input x_i, used only by
 *     position i's own attention, and a persistent pair from the output z_i,
 *     stored for every later position;
 *   - summary section 4.1: the naive schedule -- position t attends to all
 *     persistent pairs 1..t-1 that exist when it is reached.
 * The oracle runs exactly that naive schedule. Where the pages leave a step
 * open, the readings taken are:
 *   - the persistent pair is k_t = W_k RMS(z_t), v_t = W_v RMS(z_t), the same
 *     function that forms the ephemeral pair, applied to the output
 *     (kv_source_norm = 1); the text of section 2.2 breaks off before this
 *     formula, and with kv_source_norm = 0 the oracle takes the literal
 *     reading k_t = W_k z_t, v_t = W_v z_t instead;
 *   - scores are scaled by a softmax scale sigma (the pages write none and
 *     use query/key normalisation instead; sigma = 1/sqrt(head_dim) is used
 *     by the workloads, sigma = 1 gives the written operator);
 *   - RMS(v) = g * v / sqrt(mean(v^2) + eps) with a gain vector g;
 *   - the MLP is W_2 GELU(W_1 u), GELU(u) = u/2 (1 + erf(u/sqrt 2)), no biases;
 *   - residual branches are multiplied by a residual scale rho (1/sqrt(L) in
 *     the paper's parameterisation, 1 in the workloads).
 * Arithmetic is IEEE double throughout (inputs arrive as fp32 values).
 * With round_bf16 set, every tensor that the bf16 implementation holds in
 * bf16 between steps (q, k', v', the attention output, the MLP hidden
 * activation, z, and the persistent k, v) is rounded to the nearest bf16
 * value, ties to even, and the rounded values are what later steps read.
 * The residual stream h stays unrounded (it is kept in fp32), but the MLP's
 * first product reads it as a bf16 operand: W_1 RMS(h) is formed as
 * (W_1 bf16(h)) / rms(h), with rms taken from the unrounded h.
 * Reported outputs are the values BEFORE their own rounding.
 *
 * Parity of the whole layer is pinned only through its parts and special
 * cases (no numeric worked example is printed on the pages).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define RTO_OK 0
#define RTO_BAD_ARG 1
#define RTO_NO_MEMORY 2

/* ---- bf16 rounding, written from the format: 1 sign, 8 exponent bits with
 * the binary32 range, 7 stored fraction bits (8 significant bits). ------- */
double rto_round_bf16(double v) {
    if (v != v || v == 0.0 || isinf(v)) return v;
    double a = fabs(v);
    int e;
    frexp(a, &e);                       /* a = f * 2^e with f in [0.5, 1) */
    int ulp_exp = e - 8;                /* spacing of 8-significant-bit numbers */
    if (ulp_exp < -133) ulp_exp = -133; /* subnormal spacing: 2^-126 * 2^-7 */
    double r = ldexp(nearbyint(ldexp(a, -ulp_exp)), ulp_exp); /* ties to even */
    const double max_finite = ldexp(255.0, 120);              /* (2 - 2^-7) * 2^127 */
    if (r > max_finite) r = INFINITY;
    return copysign(r, v);
}

/* Threads the oracle's parallel loops use. */
int rto_num_threads(void) { return omp_get_max_threads(); }

static double keep(double v, int round_bf16) { return round_bf16 ? rto_round_bf16(v) : v; }

/* ---- sub-operations ---------------------------------------------------- */

/* RMS normalisation with gain: out_i = g_i * x_i / sqrt(mean(x^2) + eps). */
void rto_rmsnorm(const double* x, int n, const float* g, double eps, double* out) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; ++i) out[i] = (g ? (double)g[i] : 1.0) * x[i] * r;
}

/* GELU with the exact Gaussian CDF. */
double rto_gelu(double u) { return 0.5 * u * (1.0 + erf(u / sqrt(2.0))); }

/* One weight row against R vectors: y[r*ys] = sum_i w[i] U[r*us + i], each sum
 * taken in index order (rows go in chunks of 8 only so that the independent
 * sums of different rows proceed side by side). */
static void dot_rows(const float* w, int n_in, const double* U, size_t us, int R, double* y, size_t ys) {
    for (int r0 = 0; r0 < R; r0 += 8) {
        const int nr = R - r0 < 8 ? R - r0 : 8;
        double s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int i = 0; i < n_in; ++i) {
            const double wi = (double)w[i];
            for (int r = 0; r < nr; ++r) s[r] += wi * U[(size_t)(r0 + r) * us + i];
        }
        for (int r = 0; r < nr; ++r) y[(size_t)(r0 + r) * ys] = s[r];
    }
}

/*
 * One query against the key/value sequence (k_1,v_1)..(k_n,v_n) followed by
 * the ephemeral pair (k_e, v_e): the softmax-weighted average of the values
 * with weights exp(sigma <k, q>). Keys and values of the persistent part are
 * read with a stride between positions. The maximum score is subtracted
 * before exponentiating (it cancels in the ratio).
 */
static void attend(const double* q, int dh, double sigma,
                   const double* k, const double* v, size_t stride, int n,
                   const double* k_e, const double* v_e, double* s_buf, double* out) {
    double mx = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int e = 0; e < dh; ++e) s += q[e] * k[(size_t)j * stride + e];
        s_buf[j] = sigma * s;
        if (s_buf[j] > mx) mx = s_buf[j];
    }
    double se = 0.0;
    for (int e = 0; e < dh; ++e) se += q[e] * k_e[e];
    se *= sigma;
    if (se > mx) mx = se;
    double den = 0.0;
    for (int e = 0; e < dh; ++e) out[e] = 0.0;
    for (int j = 0; j < n; ++j) {
        double w = exp(s_buf[j] - mx);
        den += w;
        for (int e = 0; e < dh; ++e) out[e] += w * v[(size_t)j * stride + e];
    }
    double we = exp(se - mx);
    den += we;
    for (int e = 0; e < dh; ++e) out[e] = (out[e] + we * v_e[e]) / den;
}

/*
 * Attention of the RT layer on given tensors (naive schedule): for every
 * position t (1-based), row and head, position t's query attends to the
 * persistent pairs of positions 1..t-1 and to its own ephemeral pair.
 * All tensors are [n_pos][n_rows][n_heads][head_dim]; inputs fp32, output
 * double. Work is split over (row, head) pairs, which are independent.
 */
int rto_attention(int n_pos, int n_rows, int n_heads, int head_dim, double sigma,
                  const float* q, const float* k_eph, const float* v_eph,
                  const float* k, const float* v, double* a) {
    if (n_pos < 0 || n_rows < 0 || n_heads <= 0 || head_dim <= 0) return RTO_BAD_ARG;
    if (!q || !k_eph || !v_eph || !k || !v || !a) return RTO_BAD_ARG;
    const int d = n_heads * head_dim;
    const size_t stride = (size_t)n_rows * d; /* distance between positions */
    int status = RTO_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int p = 0; p < n_rows * n_heads; ++p) {
        const int r = p / n_heads, h = p % n_heads;
        double* kk = malloc(sizeof(double) * (size_t)n_pos * head_dim);
        double* vv = malloc(sizeof(double) * (size_t)n_pos * head_dim);
        double* s = malloc(sizeof(double) * (size_t)(n_pos + 1));
        double qq[512], ke[512], ve[512];
        if (!kk || !vv || !s || head_dim > 512) {
#pragma omp atomic write
            status = RTO_NO_MEMORY;
        } else {
            const size_t base = (size_t)r * d + (size_t)h * head_dim;
            for (int j = 0; j < n_pos; ++j)
                for (int e = 0; e < head_dim; ++e) {
                    kk[(size_t)j * head_dim + e] = k[(size_t)j * stride + base + e];
                    vv[(size_t)j * head_dim + e] = v[(size_t)j * stride + base + e];
                }
            for (int t = 0; t < n_pos; ++t) {
                const size_t off = (size_t)t * stride + base;
                for (int e = 0; e < head_dim; ++e) {
                    qq[e] = q[off + e];
                    ke[e] = k_eph[off + e];
                    ve[e] = v_eph[off + e];
                }
                attend(qq, head_dim, sigma, kk, vv, head_dim, t, ke, ve, s, a + off);
            }
        }
        free(kk);
        free(vv);
        free(s);
    }
    return status;
}

/*
 * Gradient of the RT attention map (the naive definition above) for a given
 * output adjoint a_bar = dL/da, all [n_pos][n_rows][n_heads][head_dim]. The
 * pages state only that the backward can be batched outside the position
 * loop; this is the chain rule written out for one query t:
 *   s_i = sigma <q, k_i> (i < t),  s_e = sigma <q, k'_t>,  p = softmax(s)
 *   a   = sum_i p_i v_i + p_e v'_t
 *   D   = <a_bar, a>,  dp_i = <a_bar, v_i>,  ds_i = p_i (dp_i - D)   (same for e)
 *   v_bar_i += p_i a_bar,   v'_bar_t = p_e a_bar
 *   k_bar_i += sigma ds_i q,  k'_bar_t = sigma ds_e q,
 *   q_bar_t  = sigma (sum_i ds_i k_i + ds_e k'_t).
 * Outputs are fp64 and fully written.
 */
int rto_attention_backward(int n_pos, int n_rows, int n_heads, int head_dim, double sigma,
                           const float* q, const float* k_eph, const float* v_eph,
                           const float* k, const float* v, const float* a_bar,
                           double* q_bar, double* k_eph_bar, double* v_eph_bar, double* k_bar, double* v_bar) {
    if (n_pos < 0 || n_rows < 0 || n_heads <= 0 || head_dim <= 0 || head_dim > 512) return RTO_BAD_ARG;
    if (!q || !k_eph || !v_eph || !k || !v || !a_bar || !q_bar || !k_eph_bar || !v_eph_bar || !k_bar || !v_bar)
        return RTO_BAD_ARG;
    const int d = n_heads * head_dim, dh = head_dim;
    const size_t stride = (size_t)n_rows * d;
    int status = RTO_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int pr = 0; pr < n_rows * n_heads; ++pr) {
        const int r = pr / n_heads, h = pr % n_heads;
        const size_t base = (size_t)r * d + (size_t)h * dh;
        double* p = malloc(sizeof(double) * (size_t)(n_pos + 1));
        if (!p) {
#pragma omp atomic write
            status = RTO_NO_MEMORY;
            continue;
        }
        for (int t = 0; t < n_pos; ++t)
            for (int e = 0; e < dh; ++e) {
                k_bar[(size_t)t * stride + base + e] = 0.0;
                v_bar[(size_t)t * stride + base + e] = 0.0;
            }
        for (int t = 0; t < n_pos; ++t) {
            const size_t ot = (size_t)t * stride + base;
            const float *qt = q + ot, *ket = k_eph + ot, *vet = v_eph + ot, *abt = a_bar + ot;
            /* probabilities over persistent pairs 0..t-1 (p[0..t-1]) and the ephemeral pair (p[t]) */
            double mx = -INFINITY;
            for (int i = 0; i <= t; ++i) {
                const float* ki = i < t ? k + (size_t)i * stride + base : ket;
                double sd = 0.0;
                for (int e = 0; e < dh; ++e) sd += (double)qt[e] * ki[e];
                p[i] = sigma * sd;
                if (p[i] > mx) mx = p[i];
            }
            double den = 0.0;
            for (int i = 0; i <= t; ++i) {
                p[i] = exp(p[i] - mx);
                den += p[i];
            }
            for (int i = 0; i <= t; ++i) p[i] /= den;
            /* D = <a_bar, a> with a = sum_i p_i v_i */
            double D = 0.0;
            for (int i = 0; i <= t; ++i) {
                const float* vi = i < t ? v + (size_t)i * stride + base : vet;
                double dpi = 0.0;
                for (int e = 0; e < dh; ++e) dpi += (double)abt[e] * vi[e];
                D += p[i] * dpi;
            }
            double* qb = q_bar + ot;
            for (int e = 0; e < dh; ++e) qb[e] = 0.0;
            for (int i = 0; i <= t; ++i) {
                const int eph = i == t;
                const float* ki = eph ? ket : k + (size_t)i * stride + base;
                const float* vi = eph ? vet : v + (size_t)i * stride + base;
                double* kb = eph ? k_eph_bar + ot : k_bar + (size_t)i * stride + base;
                double* vb = eph ? v_eph_bar + ot : v_bar + (size_t)i * stride + base;
                double dpi = 0.0;
                for (int e = 0; e < dh; ++e) dpi += (double)abt[e] * vi[e];
                const double ds = p[i] * (dpi - D);
                for (int e = 0; e < dh; ++e) {
                    if (eph) {
                        kb[e] = sigma * ds * qt[e];
                        vb[e] = p[i] * abt[e];
                    } else {
                        kb[e] += sigma * ds * qt[e];
                        vb[e] += p[i] * abt[e];
                    }
                    qb[e] += sigma * ds * ki[e];
                }
            }
        }
        free(p);
    }
    return status;
}

/*
 * The same attention for selected positions only: a_sel[i] is the output of
 * position sel[i] (1-based), [n_sel][n_rows][n_heads][head_dim]. Position t
 * reads the persistent pairs 1..t-1 and its own ephemeral pair, so any
 * position can be computed alone.
 */
int rto_attention_at(int n_pos, int n_rows, int n_heads, int head_dim, double sigma,
                     const float* q, const float* k_eph, const float* v_eph,
                     const float* k, const float* v, int n_sel, const int* sel, double* a_sel) {
    if (n_pos < 0 || n_rows < 0 || n_heads <= 0 || head_dim <= 0 || head_dim > 512 || n_sel < 0) return RTO_BAD_ARG;
    if (!q || !k_eph || !v_eph || !k || !v || !a_sel || (n_sel && !sel)) return RTO_BAD_ARG;
    for (int i = 0; i < n_sel; ++i)
        if (sel[i] < 1 || sel[i] > n_pos) return RTO_BAD_ARG;
    const int d = n_heads * head_dim;
    const size_t stride = (size_t)n_rows * d;
    int status = RTO_OK;
#pragma omp parallel for schedule(dynamic, 1) collapse(2)
    for (int i = 0; i < n_sel; ++i) {
        for (int p = 0; p < n_rows * n_heads; ++p) {
            const int t = sel[i] - 1, r = p / n_heads, h = p % n_heads;
            const size_t base = (size_t)r * d + (size_t)h * head_dim;
            double* kk = malloc(sizeof(double) * ((size_t)t * head_dim + 1));
            double* vv = malloc(sizeof(double) * ((size_t)t * head_dim + 1));
            double* s = malloc(sizeof(double) * (size_t)(t + 1));
            double qq[512], ke[512], ve[512];
            if (!kk || !vv || !s) {
#pragma omp atomic write
                status = RTO_NO_MEMORY;
            } else {
                for (int j = 0; j < t; ++j)
                    for (int e = 0; e < head_dim; ++e) {
                        kk[(size_t)j * head_dim + e] = k[(size_t)j * stride + base + e];
                        vv[(size_t)j * head_dim + e] = v[(size_t)j * stride + base + e];
                    }
                const size_t off = (size_t)t * stride + base;
                for (int e = 0; e < head_dim; ++e) {
                    qq[e] = q[off + e];
                    ke[e] = k_eph[off + e];
                    ve[e] = v_eph[off + e];
                }
                attend(qq, head_dim, sigma, kk, vv, head_dim, t, ke, ve, s,
                       a_sel + (size_t)i * stride + base);
            }
            free(kk);
            free(vv);
            free(s);
        }
    }
    return status;
}

/* ---- the layer ---------------------------------------------------------- */

typedef struct {
    int32_t n_pos, n_rows, d_model, n_heads, head_dim, d_ff;
    double softmax_scale, residual_scale, rms_eps;
    int32_t kv_from_input; /* 0: persistent pair from z_t (RT); 1: from x_t (Transformer) */
    int32_t round_bf16;    /* round the stored tensors to bf16 */
    int32_t qk_norm;       /* RMS-normalise each head's query and key (ephemeral and persistent) */
    int32_t kv_source_norm;/* RT: 1 the persistent pair reads RMS_attn(z_t); 0 it reads z_t itself */
} rto_layer_cfg;

typedef struct {
    const float *w_q, *w_k, *w_v, *w_o; /* [d][d], row-major [out][in] */
    const float *w_1;                   /* [F][d] */
    const float *w_2;                   /* [d][F] */
    const float *g_attn, *g_mlp;        /* [d]; NULL means ones */
    const float *g_q, *g_k;             /* [d] query / key norm gains (qk_norm); NULL means ones */
} rto_weights;

/* Outputs, each [n_pos][n_rows][width], values before their own rounding.
 * Any pointer may be NULL except x_next. */
typedef struct {
    double *z, *k, *v;        /* layer output and persistent pair, width d */
    double *q, *k_eph, *v_eph;/* width d */
    double *a;                /* attention output, all heads, width d */
    double *h;                /* x + rho W_o a, width d */
    double *g;                /* MLP hidden activation GELU(W_1 RMS(h)), width F */
    float *x_next;            /* z as stored (rounded when round_bf16): the next layer's input */
} rto_layer_out;

static void put(double* dst, size_t off, const double* src, int n) {
    if (dst) memcpy(dst + off, src, sizeof(double) * (size_t)n);
}

/*
 * The RT layer over positions 1..n_pos (naive schedule), for n_rows
 * independent batch rows, input x [n_pos][n_rows][d]. Per position t and
 * row (translated paper sections 2.1-2.2):
 *   u      = RMS_attn(x_t)
 *   q, k', v' = W_q u, W_k u, W_v u
 *   a_h    = Attn((k_1,v_1)..(k_{t-1},v_{t-1}), (k'_h, v'_h); q_h) per head h
 *   h      = x_t + rho W_o a
 *   z_t    = h + rho W_2 GELU(W_1 RMS_mlp(h))
 *   k_t, v_t = W_k RMS_attn(z_t), W_v RMS_attn(z_t)   (from x_t instead when
 *            kv_from_input is set, which is the standard Transformer layer;
 *            W_k z_t, W_v z_t when kv_source_norm is 0)
 * With qk_norm, every query and key (q, k', k) is RMS-normalised per head
 * after its projection, with gains g_q, g_k (the "magenta" RMS of the
 * translated paper's section 2 notation, read per head as in the query/key
 * normalisation it cites).
 * Positions run in order; rows are independent, and the work inside each
 * position is split over rows and output features.
 */
int rto_layer_forward(const rto_layer_cfg* c, const rto_weights* w, const float* x, rto_layer_out* out) {
    if (!c || !w || !x || !out || !out->x_next) return RTO_BAD_ARG;
    const int N = c->n_pos, R = c->n_rows, d = c->d_model, H = c->n_heads, dh = c->head_dim, F = c->d_ff;
    if (N < 0 || R < 0 || d <= 0 || H <= 0 || dh <= 0 || F <= 0 || H * dh != d || dh > 512) return RTO_BAD_ARG;
    if (!w->w_q || !w->w_k || !w->w_v || !w->w_o || !w->w_1 || !w->w_2) return RTO_BAD_ARG;
    const int rb = c->round_bf16;
    const double sigma = c->softmax_scale, rho = c->residual_scale, eps = c->rms_eps;
    const size_t Rd = (size_t)R * d;

    /* persistent keys/values as stored: [n_pos][R][d] */
    double* Kc = malloc(sizeof(double) * (size_t)N * Rd + 1);
    double* Vc = malloc(sizeof(double) * (size_t)N * Rd + 1);
    /* per-row scratch for one position */
    double* buf = malloc(sizeof(double) * (size_t)R * (10 * (size_t)d + 2 * (size_t)F));
    if (!Kc || !Vc || !buf) {
        free(Kc); free(Vc); free(buf);
        return RTO_NO_MEMORY;
    }
    const size_t per_row = 10 * (size_t)d + 2 * (size_t)F;

    for (int t = 0; t < N; ++t) {
        /* 1. projections of the input: u, q, k', v' */
#pragma omp parallel for schedule(static)
        for (int r = 0; r < R; ++r) {
            double* b = buf + r * per_row;
            double *xt = b, *u = b + d;
            for (int i = 0; i < d; ++i) xt[i] = x[(size_t)t * Rd + (size_t)r * d + i];
            rto_rmsnorm(xt, d, w->g_attn, eps, u);
        }
#pragma omp parallel for schedule(static)
        for (int o = 0; o < 3 * d; ++o) {
            const int which = o / d, oo = o % d;
            const float* W = which == 0 ? w->w_q : (which == 1 ? w->w_k : w->w_v);
            /* q at 2d, k' at 3d, v' at 4d of each row's scratch */
            dot_rows(W + (size_t)oo * d, d, buf + d, per_row, R, buf + 2 * d + o, per_row);
        }
        if (c->qk_norm) {
#pragma omp parallel for schedule(static)
            for (int r = 0; r < R; ++r) {
                double* b = buf + r * per_row;
                for (int hh = 0; hh < H; ++hh) {
                    double* qh = b + 2 * d + hh * dh;
                    double* kh = b + 3 * d + hh * dh;
                    rto_rmsnorm(qh, dh, w->g_q ? w->g_q + hh * dh : NULL, eps, qh);
                    rto_rmsnorm(kh, dh, w->g_k ? w->g_k + hh * dh : NULL, eps, kh);
                }
            }
        }
        /* 2. attention of position t over persistent pairs 1..t-1 plus its own ephemeral pair */
#pragma omp parallel for schedule(dynamic, 1)
        for (int p = 0; p < R * H; ++p) {
            const int r = p / H, hh = p % H;
            double* b = buf + r * per_row;
            double qh[512], ke[512], ve[512];
            double* s = malloc(sizeof(double) * (size_t)(t + 1));
            if (!s) abort(); /* a few KB; the oracle has no recovery path */
            for (int e = 0; e < dh; ++e) {
                qh[e] = keep(b[2 * d + hh * dh + e], rb);
                ke[e] = keep(b[3 * d + hh * dh + e], rb);
                ve[e] = keep(b[4 * d + hh * dh + e], rb);
            }
            const size_t base = (size_t)r * d + (size_t)hh * dh;
            attend(qh, dh, sigma, Kc + base, Vc + base, Rd, t, ke, ve, s, b + 5 * d + hh * dh);
            free(s);
        }
        /* 3. output projection + residual: h = x_t + rho W_o a (a read as stored) */
        for (int r = 0; r < R; ++r) {
            double* b = buf + r * per_row;
            for (int i = 0; i < d; ++i) b[9 * d + i] = keep(b[5 * d + i], rb);
        }
#pragma omp parallel for schedule(static)
        for (int o = 0; o < d; ++o) {
            double s[256];
            for (int r0 = 0; r0 < R; r0 += 256) {
                const int nr = R - r0 < 256 ? R - r0 : 256;
                dot_rows(w->w_o + (size_t)o * d, d, buf + (size_t)r0 * per_row + 9 * d, per_row, nr, s, 1);
                for (int r = 0; r < nr; ++r) {
                    double* b = buf + (size_t)(r0 + r) * per_row;
                    b[6 * d + o] = b[o] + rho * s[r]; /* h */
                }
            }
        }
        /* 4. MLP on RMS_mlp(h): g = GELU(W_1 u2), z = h + rho W_2 g */
#pragma omp parallel for schedule(static)
        for (int r = 0; r < R; ++r) {
            double* b = buf + r * per_row;
            if (rb) {
                /* RMS of the unrounded h; the product reads h rounded to bf16 */
                double ss = 0.0;
                for (int i = 0; i < d; ++i) ss += b[6 * d + i] * b[6 * d + i];
                const double rr = 1.0 / sqrt(ss / d + eps);
                for (int i = 0; i < d; ++i)
                    b[7 * d + i] = (w->g_mlp ? (double)w->g_mlp[i] : 1.0) * rto_round_bf16(b[6 * d + i]) * rr;
            } else {
                rto_rmsnorm(b + 6 * d, d, w->g_mlp, eps, b + 7 * d);
            }
        }
#pragma omp parallel for schedule(static)
        for (int o = 0; o < F; ++o) {
            dot_rows(w->w_1 + (size_t)o * d, d, buf + 7 * d, per_row, R, buf + 10 * d + o, per_row);
            for (int r = 0; r < R; ++r) {
                double* b = buf + (size_t)r * per_row;
                b[10 * d + o] = rto_gelu(b[10 * d + o]);      /* g before rounding */
                b[10 * d + F + o] = keep(b[10 * d + o], rb);   /* g as stored */
            }
        }
#pragma omp parallel for schedule(static)
        for (int o = 0; o < d; ++o) {
            double s[256];
            for (int r0 = 0; r0 < R; r0 += 256) {
                const int nr = R - r0 < 256 ? R - r0 : 256;
                dot_rows(w->w_2 + (size_t)o * F, F, buf + (size_t)r0 * per_row + 10 * d + F, per_row, nr, s, 1);
                for (int r = 0; r < nr; ++r) {
                    double* b = buf + (size_t)(r0 + r) * per_row;
                    b[8 * d + o] = b[6 * d + o] + rho * s[r]; /* z before rounding */
                }
            }
        }
        /* 5. persistent pair of position t, from the stored output (or the input) */
#pragma omp parallel for schedule(static)
        for (int r = 0; r < R; ++r) {
            double* b = buf + r * per_row;
            double* zs = b + 7 * d; /* reuse: z as stored, then its RMS */
            for (int i = 0; i < d; ++i) {
                double zv = keep(b[8 * d + i], rb);
                out->x_next[(size_t)t * Rd + (size_t)r * d + i] = (float)zv;
                zs[i] = c->kv_from_input ? b[i] : zv;
            }
            if (c->kv_from_input || c->kv_source_norm) rto_rmsnorm(zs, d, w->g_attn, eps, zs);
        }
#pragma omp parallel for schedule(static)
        for (int o = 0; o < 2 * d; ++o) {
            const int oo = o % d;
            double s[256];
            for (int r0 = 0; r0 < R; r0 += 256) {
                const int nr = R - r0 < 256 ? R - r0 : 256;
                dot_rows((o < d ? w->w_k : w->w_v) + (size_t)oo * d, d, buf + (size_t)r0 * per_row + 7 * d,
                         per_row, nr, s, 1);
                for (int r = 0; r < nr; ++r) {
                    const size_t off = (size_t)t * Rd + (size_t)(r0 + r) * d + oo;
                    if (o < d) {
                        buf[(size_t)(r0 + r) * per_row + 9 * d + oo] = s[r]; /* k, finished below */
                    } else {
                        if (out->v) out->v[off] = s[r];
                        Vc[off] = keep(s[r], rb);
                    }
                }
            }
        }
#pragma omp parallel for schedule(static)
        for (int r = 0; r < R; ++r) {
            double* kr = buf + r * per_row + 9 * d;
            if (c->qk_norm)
                for (int hh = 0; hh < H; ++hh)
                    rto_rmsnorm(kr + hh * dh, dh, w->g_k ? w->g_k + hh * dh : NULL, eps, kr + hh * dh);
            for (int i = 0; i < d; ++i) {
                const size_t off = (size_t)t * Rd + (size_t)r * d + i;
                if (out->k) out->k[off] = kr[i];
                Kc[off] = keep(kr[i], rb);
            }
        }
        /* 6. report */
        for (int r = 0; r < R; ++r) {
            double* b = buf + r * per_row;
            const size_t off = (size_t)t * Rd + (size_t)r * d;
            put(out->q, off, b + 2 * d, d);
            put(out->k_eph, off, b + 3 * d, d);
            put(out->v_eph, off, b + 4 * d, d);
            put(out->a, off, b + 5 * d, d);
            put(out->h, off, b + 6 * d, d);
            put(out->z, off, b + 8 * d, d);
            if (out->g) memcpy(out->g + (size_t)t * R * F + (size_t)r * F, b + 10 * d, sizeof(double) * F);
        }
    }
    free(Kc);
    free(Vc);
    free(buf);
    return RTO_OK;
}
