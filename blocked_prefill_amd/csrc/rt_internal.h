// Host-side internal interfaces of the library (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rt_prefill.h"

namespace rt {

constexpr float kLog2eHost = 1.4426950408889634f;  // log2(e): scores are kept in base 2

// One step of the blocked schedule applied to a contiguous range of query
// rows, optionally finishing the first row of the range into a_out.
// Row indices are 0-based (row r holds position r+1).
struct UpdateArgs {
    const void* q;      // [N][P][dh]
    const void* k;      // [N][P][dh] persistent keys
    const void* v;      // [N][P][dh] persistent values
    const void* k_eph;  // [N][P][dh] (read only when fin)
    const void* v_eph;  // [N][P][dh] (read only when fin)
    float* m;           // [N][P]
    float* l;           // [N][P]
    float* o;           // [N][P][dh]
    void* a_out;        // [P][dh] (written only when fin)
    int64_t P;          // batch * n_heads
    int32_t kv0;        // first KV row of the block
    int32_t nkv;        // KV rows in the block (0: finalize only)
    int32_t q0;         // first query row
    int32_t nq;         // query rows
    float sigma2;       // softmax_scale * log2(e)
    int32_t init;       // state rows are initialised, not read (first touch)
    int32_t fin;        // row q0 is finished into a_out and its state is not written
    float* lse;         // [N][P] (nullable): base-2 log-sum-exp of the finished row, m + log2(l)
    // Several steps of one level in one launch (every pair known up front):
    // n_steps steps, step s applying keys kv0 + 2s*nkv.. to queries q0 + 2s*nkv..
    // (query count clipped at n_pos; only step 0 initialises its rows; step s
    // finishes into a_out + s*a_step bytes). 0 or 1: one step.
    int32_t n_steps;
    int32_t n_pos;
    int64_t a_step;
};

hipError_t launch_update(rt_dtype dt, int head_dim, const UpdateArgs& a, hipStream_t s);
// n blocked steps of 1, 2 or 4 pairs (all the same length, the same pair count;
// bf16, head_dim 64), kMaxUpdateGroup per launch: the small steps of the layers
// of a stack.
constexpr int kMaxUpdateGroup = 8;
hipError_t launch_update_small_group(rt_dtype dt, int head_dim, const UpdateArgs* us, int n, hipStream_t s);
// Plain causal attention over nq positions: query row i attends key/value rows
// 0..i of k/v and is written to row i of a_out ([nq][P][dh]); m/l/o unused.
hipError_t launch_causal_attention(rt_dtype dt, int head_dim, const UpdateArgs& a, hipStream_t s);

// Attention backward of the blocked schedule (see backward.hip). Tensors as
// in UpdateArgs; adjoints and outputs fp32 [N][P][dh], lse/delta fp32 [N][P].
struct BackwardArgs {
    const void *q, *k_eph, *v_eph, *k, *v, *a;  // dtype
    const float* lse;                           // base-2 log-sum-exp of every query
    const float* a_bar;                         // output adjoint
    float *q_bar, *k_eph_bar, *v_eph_bar, *k_bar, *v_bar;
    float* delta;                               // <a_bar, a> per query (written by the first pass)
    int64_t P;
    int32_t n_pos;
    float sigma;                                // softmax_scale (natural units)
    float sigma2;                               // softmax_scale * log2(e)
    int32_t kv_accumulate;                      // 0: a step sets its block's last k_bar/v_bar row (forward
                                                // step order); 1: every row accumulates (rows pre-zeroed)
};
// Per-query pass over all positions: delta, the ephemeral pair's gradients, q_bar's ephemeral term.
hipError_t launch_backward_prep(rt_dtype dt, int head_dim, const BackwardArgs& b, hipStream_t s);
// Step t of the blocked schedule, reversed: the block of keys (kv0, kv0+nkv] against the queries
// (q0, q0+nq]; k_bar/v_bar rows of the block accumulate (row kv0+nkv-1, first touched here when
// steps run in forward order, is set unless kv_accumulate), q_bar rows of the queries accumulate.
hipError_t launch_backward_step(rt_dtype dt, int head_dim, const BackwardArgs& b, int32_t kv0, int32_t nkv,
                                int32_t q0, int32_t nq, hipStream_t s);
// Zero rows [row0, row0 + rows) of k_bar and v_bar (pairs no query reads).
hipError_t launch_backward_zero_rows(int head_dim, const BackwardArgs& b, int32_t row0, int32_t rows, hipStream_t s);

// C[M][N] = epilogue(A[M][K] * W^T), W given as up to 3 column segments of
// seg_n rows each ([seg_n][K] row-major), outputs likewise split.
enum : int {
    EPI_RMS = 1,        // scale rows by 1/rms of the A row, summed by this kernel
    EPI_GELU = 2,       // GELU (erf form)
    EPI_RESID = 4,      // C = R + rscale * acc
    EPI_RMS_PARTS = 8,  // scale rows by 1/rms from n_parts partial sums of squares (rss_in)
    EPI_ROWSS = 16,     // write this tile's partial sum of squares of each stored row (rss_out)
    EPI_COPY = 32,      // also store the result as bf16 into C2
    EPI_QKNORM = 64,    // RMS-normalise each head_dim-wide head of the segments in qkn_mask
    EPI_PAIRKV = 128,   // tile n holds columns n*BN/2.. of segment 0 (left half) and of segment 1 (right)
    EPI_UPDATE = 256,   // (with EPI_PAIRKV, bf16, head_dim 64) then run upd, a small blocked step whose
                        // newest key/value row is this product's output (see gemm.hip)
    EPI_DGELU = 512,    // multiply by GELU'(R[row][col]) (the backward through the MLP's activation)
    // kernel shape (not epilogue) flags, bf16 pipelined kernel:
    PIPE_DMA = 1024,    // K tiles go straight from global memory into a ring of D LDS stages
                        // (global_load_lds), no register staging; one K group
    PIPE_XCD = 2048,    // grouped launch: the workgroups an XCD runs take one contiguous range of
                        // (product, row tile, column tile), so a weight slab and an A row block are
                        // each fetched into few XCDs' L2
};
struct GemmArgs {
    const void* A;      // [M][lda]
    int64_t lda;
    const void* W[3];   // [seg_n][K] each
    void* C[3];         // [M][ldc] each
    int64_t ldc;
    int32_t seg_n;
    const void* R;      // [M][ldr] residual, added as R + rscale * acc
    int64_t ldr;
    float rscale;
    float eps;
    int64_t M;
    int32_t N, K;
    // Columns of A (0: K). When a_k < K, column k of the product reads column
    // k mod a_k of A: a bf16 weight whose RMS gain is folded in is stored as
    // two bf16 halves side by side ([rows][2 a_k]: the rounded product, then
    // its rounding error), and both halves multiply the same A row. The RMS
    // of an A row is taken over a_k columns.
    int32_t a_k;
    int64_t ldw;          // row stride of W (0: K)
    int32_t no_rms;       // 1: EPI_RMS / EPI_RMS_PARTS scale rows by 1 (a persistent pair read from z itself)
    const float* rss_in;  // [M][n_parts] (EPI_RMS_PARTS), n_parts % 4 == 0, <= 64
    int32_t n_parts;
    float* rss_out;       // [M][N / tile width] (EPI_ROWSS)
    void* C2;             // [M][ldc] bf16 (EPI_COPY)
    int32_t qkn_mask;            // bit s: normalise segment s per head (query/key norm); 0: none
    int32_t head_dim;            // head width of that norm
    const float* qkn_gain[3];    // [seg_n] gains per segment (nullptr: ones)
    UpdateArgs upd;              // EPI_UPDATE: the step (block of 1, 2 or 4 pairs ending at this row)
};
// Column-tile width of the GEMMs whose epilogue writes row partial sums
// (the number of partial sums per row is N / this width).
constexpr int kRowSSTile = 32;
// Kinds of GEMM, by operand/output element types.
enum class GemmKind {
    QKV,      // A = x (T), RMS, C = q|k'|v' (T)
    WO,       // A = a (T), C = h (f32), R = x (T)
    W1,       // A = h (f32), RMS + GELU, C = g (T)
    W2,       // A = g (T), C = z (T), R = h (f32)
    KV,       // A = z (T), RMS, C = k|v (T)
    KV_UPDATE,// KV (bf16, head_dim 64), then the small blocked step g.upd fused into the same launch
    W1_PRE,   // A = h (bf16 copy with RMS partials, or fp32), RMS, C = W_1 RMS(h) before the GELU (T)
    PLAIN,    // C (fp32) = A (T) * W^T, no epilogue (the backward's adjoint products)
    W2_BWD,   // C (T) = (A * W^T) * GELU'(R), R = the MLP's pre-activation (T); per-position rows only
    WGRAD,    // C (fp32) = A * W^T with a long K (a weight gradient's reduction over rows; W row stride ldw)
};
hipError_t launch_gemm(rt_dtype dt, GemmKind kind, const GemmArgs& g, hipStream_t s);
// n products of one kind and shape (the same N, K and epilogue inputs; row
// counts may differ) in as few launches as possible, kMaxGemmGroup per launch
// (bf16; fp32 products run one launch each).
constexpr int kMaxGemmGroup = 8;
hipError_t launch_gemm_group(rt_dtype dt, GemmKind kind, const GemmArgs* gs, int n, hipStream_t s);
// `splits` products in one launch that differ only in their K range (WGRAD): product z reads A and W
// from column z * k_step on (elements) and writes C from element z * c_step on; g is product 0.
hipError_t launch_gemm_splitk(rt_dtype dt, GemmKind kind, const GemmArgs& g, int splits, int64_t k_step,
                              int64_t c_step, hipStream_t s);
// out[row][0..3] = sums of x[row][c]^2 over the four quarters of the row (D % 32 == 0); a QKV
// product given them (rss_in, n_parts = 4) takes its RMS from them.
hipError_t launch_row_sumsq(rt_dtype dt, const void* x, int64_t rows, int D, float* out, hipStream_t s);

// ---- the layer backward's pieces (layer_backward.hip)
// dst[c][col0 + r] = src[r][c] for src [rows][cols] (dtype dt), dst row stride ldd.
hipError_t launch_transpose(rt_dtype dt, const void* src, int64_t rows, int64_t cols, void* dst, int64_t ldd,
                            int64_t col0, hipStream_t s);
// dst[r][s*D + c] = scale * src_s[r][c] for s < nsrc (fp32 sources [rows][D], dst dtype dt, row stride ldd).
hipError_t launch_pack(rt_dtype dt, void* dst, int64_t ldd, const float* s0, const float* s1, const float* s2,
                       int nsrc, int64_t rows, int D, float scale, hipStream_t s);
// Per row of x [rows][D]: out = base + the adjoint of x for y = g x / rms(x) given y_bar
// (base, g may be null: 0, ones); out2 (nullable) = scale2 * out in out2_dt; rinv_out (nullable) = 1/rms.
hipError_t launch_rms_bwd(rt_dtype x_dt, rt_dtype out2_dt, const void* x, const float* ybar, const float* g,
                          float eps, const float* base, float* out, void* out2, float scale2, float* rinv_out,
                          int64_t rows, int D, hipStream_t s);
// out = g x / rms(x) per row, in out_dt.
hipError_t launch_rms_apply(rt_dtype x_dt, rt_dtype out_dt, const void* x, const float* g, float eps, void* out,
                            int64_t rows, int D, hipStream_t s);
// u = GELU(u) in place.
hipError_t launch_gelu_inplace(rt_dtype dt, void* u, int64_t n, hipStream_t s);
// Gain gradient: out[c] (+)= sum_r y_bar[r][c] x[r][c] rinv[r]; part holds gain_grad_blocks(rows) * D floats.
constexpr int kGainRowsPerBlock = 256;  // rows per first-level block
constexpr int kGainGroup = 64;          // first-level blocks per second-level sum
int64_t gain_grad_blocks(int64_t rows);
hipError_t launch_gain_grad(rt_dtype x_dt, const float* ybar, const void* x, const float* rinv, int64_t rows, int D,
                            float* part, float* out, int accumulate, hipStream_t s);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
// Weight gradients out[o][i] (+)= sum_r abar[r][o] u[r][i] over R rows (abar row stride lda, u row stride ldu,
// both in dt; out fp32 [O][I]; O, I multiples of 4, of 128 for bf16): both operands transposed into ws
// (ta [O][rows_pad], tu [I][rows_pad]), the product split into `splits` K ranges (fp32 partials in ws.part,
// splits * O * I floats), then added up. u_ready: ws.tu already holds this u (the previous call's).
constexpr int kWgradSplits = 16;
struct WgradPlan {
    int64_t rows_pad;  // R rounded up to 128 * splits
    int splits;
};
WgradPlan wgrad_plan(int64_t rows);
struct WgradScratch {
    void* ta;          // [max O][rows_pad] (dt)
    void* tu;          // [max I][rows_pad] (dt)
    float* part;       // [splits][max O*I]
    int64_t rows_pad;
};
hipError_t weight_grad(rt_dtype dt, const void* abar, int64_t lda, const void* u, int64_t ldu, int64_t R, int O,
                       int I, float* out, bool accumulate, bool u_ready, const WgradScratch& ws, hipStream_t s);
bool gemm_shape_supported(rt_dtype dt, int64_t M, int N, int K);

// Fold an RMS gain into the following projection, p[r][c] = W[r][c] * g[c]
// computed in fp32: fp32 layers store W_out = p ([rows][cols]); bf16 layers
// store W_out = [bf16(p) | bf16(p - bf16(p))] ([rows][2 cols]), whose sum is
// p to ~2^-17 relative (read with a_k = cols, K = 2 cols).
// The calling thread's error text (rt_last_error) set to a + b; returns st.
rt_status set_error(rt_status st, const char* a, const char* b);
// The argument checks of rt_layer_decode_step other than its workspace (no HIP call).
rt_status check_decode_args(const rt_layer_desc* desc, const rt_layer_weights* w, int32_t n_past, const void* x_t,
                            void* z_t, void* k_cache, void* v_cache);

hipError_t launch_fold_gain(rt_dtype dt, const void* W, const float* g, void* W_out, int64_t rows, int cols,
                            hipStream_t s);

}  // namespace rt
