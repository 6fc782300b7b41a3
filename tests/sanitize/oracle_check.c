/* A sanitizer build's run of the CPU oracle (test infrastructure): a small
 * layer in both storage modes, both persistent-pair readings and the
 * Transformer mode, the attention at selected positions and the attention
 * backward; exits non-zero on a bad status or a non-finite output. The
 * sanitizers abort on a memory or undefined-behaviour error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
    int32_t n_pos, n_rows, d_model, n_heads, head_dim, d_ff;
    double softmax_scale, residual_scale, rms_eps;
    int32_t kv_from_input, round_bf16, qk_norm, kv_source_norm;
} cfg_t;
typedef struct {
    const float *w_q, *w_k, *w_v, *w_o, *w_1, *w_2, *g_attn, *g_mlp, *g_q, *g_k;
} weights_t;
typedef struct {
    double *z, *k, *v, *q, *k_eph, *v_eph, *a, *h, *g;
    float* x_next;
} out_t;

int rto_layer_forward(const cfg_t*, const weights_t*, const float*, out_t*);
int rto_attention_at(int, int, int, int, double, const float*, const float*, const float*, const float*,
                     const float*, int, const int*, double*);
int rto_attention_backward(int, int, int, int, double, const float*, const float*, const float*, const float*,
                           const float*, const float*, double*, double*, double*, double*, double*);

static float* randn(size_t n, double scale, unsigned* st) {
    float* p = malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) {
        *st = *st * 1664525u + 1013904223u;
        p[i] = (float)(((double)(*st >> 8) / 16777216.0 - 0.5) * 3.4 * scale);
    }
    return p;
}

static int all_finite(const double* p, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) return 0;
    return 1;
}

int main(void) {
    const int N = 19, R = 3, d = 64, H = 2, F = 128;
    const size_t nd = (size_t)N * R * d;
    unsigned st = 12345u;
    float* x = randn(nd, 1.0, &st);
    weights_t w = {randn((size_t)d * d, 0.125, &st), randn((size_t)d * d, 0.125, &st), randn((size_t)d * d, 0.125, &st),
                   randn((size_t)d * d, 0.125, &st), randn((size_t)F * d, 0.125, &st), randn((size_t)d * F, 0.09, &st),
                   NULL, NULL, NULL, NULL};
    double *z = malloc(nd * sizeof(double)), *k = malloc(nd * sizeof(double)), *v = malloc(nd * sizeof(double));
    double* g = malloc((size_t)N * R * F * sizeof(double));
    float* xn = malloc(nd * sizeof(float));
    int bad = 0;
    for (int mode = 0; mode < 5; ++mode) {
        cfg_t c = {N, R, d, H, d / H, F, 0.17, 0.8, 1e-6, mode == 3, mode == 1 || mode == 4, mode == 4, mode != 2};
        out_t o = {z, k, v, NULL, NULL, NULL, NULL, NULL, g, xn};
        if (rto_layer_forward(&c, &w, x, &o) != 0 || !all_finite(z, nd) || !all_finite(k, nd) || !all_finite(v, nd)) {
            fprintf(stderr, "layer mode %d failed\n", mode);
            bad = 1;
        }
    }
    const int sel[3] = {1, 7, N};
    double* a = malloc(3 * (size_t)R * d * sizeof(double));
    if (rto_attention_at(N, R, H, d / H, 0.2, x, x, x, x, x, 3, sel, a) != 0 || !all_finite(a, 3 * (size_t)R * d)) {
        fprintf(stderr, "attention_at failed\n");
        bad = 1;
    }
    double* gr[5];
    for (int i = 0; i < 5; ++i) gr[i] = malloc(nd * sizeof(double));
    if (rto_attention_backward(N, R, H, d / H, 0.2, x, x, x, x, x, x, gr[0], gr[1], gr[2], gr[3], gr[4]) != 0 ||
        !all_finite(gr[3], nd)) {
        fprintf(stderr, "attention_backward failed\n");
        bad = 1;
    }
    for (int i = 0; i < 5; ++i) free(gr[i]);
    free(a); free(z); free(k); free(v); free(g); free(xn); free(x);
    free((void*)w.w_q); free((void*)w.w_k); free((void*)w.w_v); free((void*)w.w_o); free((void*)w.w_1);
    free((void*)w.w_2);
    printf("oracle_check: %s\n", bad ? "FAILED" : "ok");
    return bad;
}
