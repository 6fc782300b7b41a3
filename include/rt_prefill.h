/*
 * rt_prefill.h -- C ABI of the MI355X (gfx950) Recurrent Transformer prefill library.
 *
 * The library computes the forward pass of a Recurrent Transformer (RT)
 * layer over a whole sequence (prefill / training forward), as defined on
 * the Recurrent Transformer reading note (lshu.cn/news/403416):
 *   - translated paper section 2.2 and summary section 2.2: queries and an
 *     ephemeral key/value pair of position t come from the layer input x_t;
 *     the persistent pair (k_t, v_t) that later positions attend to comes
 *     from the layer output z_t, so pairs are revealed one position at a time;
 *   - summary section 4.2 ("blocked schedule"): every query is formed up
 *     front; each keeps an online-softmax state (running maximum m,
 *     normaliser l, numerator o); when pair t is revealed, the pairs
 *     t-b+1..t are applied to queries t+1..t+b, b the largest power of two
 *     dividing t. The result equals the naive schedule up to rounding order.
 *   - translated paper section 6.3 / summary section 5.3: tensors indexed by
 *     position are stored position-major.
 *
 * Conventions shared by every entry point
 *   - Positions are 1-based in the API (t = 1..seq_len), as on the pages.
 *   - All tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *     16-byte aligned, in the layouts stated below (row-major, last index
 *     fastest). N = seq_len, B = batch, H = n_heads, dh = head_dim,
 *     d = H*dh = d_model, F = d_ff. "[N][B][H][dh]" is the same memory as
 *     "[N][B][d]": head h of a row is columns h*dh .. h*dh+dh-1.
 *   - Element type of every activation, weight and cache tensor is the
 *     descriptor's dtype (fp32 or bf16). The online-softmax state is always
 *     fp32. Accumulation is always fp32.
 *   - Calls enqueue work on the given HIP stream (NULL = the default stream)
 *     and return without waiting; a kernel fault surfaces at the caller's next
 *     synchronisation (immediately with RT_FLAG_DEBUG_SYNC).
 *   - Arguments are validated before any HIP call. Errors are returned as
 *     rt_status, never thrown or aborted; rt_last_error() gives the text of
 *     the calling thread's last error.
 *   - The library allocates no device memory in any entry point except
 *     plan creation (rt_layer_plan_create, rt_stack_plan_create: a plan owns
 *     only its captured HIP graphs). Every product, the weight gradients
 *     included, runs in the library's own kernels: it calls no vendor GEMM
 *     library.
 */
#ifndef RT_PREFILL_H
#define RT_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* rt_stream_t; /* hipStream_t */

typedef enum {
    RT_OK = 0,
    RT_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, t out of range, misaligned pointer */
    RT_ERR_UNSUPPORTED = 2,  /* valid but not implemented: head_dim not in {32, 64, 128}, odd sizes */
    RT_ERR_WORKSPACE = 3,    /* workspace_bytes smaller than rt_layer_workspace_bytes() */
    RT_ERR_HIP = 4,          /* a HIP runtime call failed; see rt_last_error() */
    RT_ERR_INTERNAL = 5      /* an internal consistency check failed (a defect of this library) */
} rt_status;

typedef enum { RT_F32 = 0, RT_BF16 = 1 } rt_dtype;

/* flags of rt_layer_desc */
#define RT_FLAG_DEBUG_SYNC 1u   /* synchronise and check after every launch (slow; for debugging) */
/* The naive schedule (reading note, summary section 4.1): after position t,
 * query t+1 reads all persistent pairs 1..t in one pass. Same result as the
 * blocked schedule up to rounding order, with Theta(N^2) traffic; kept as
 * the comparison point of the translated paper's Figure 4. */
#define RT_FLAG_NAIVE_SCHEDULE 2u
/* The standard Transformer layer (translated paper section 2.1): the pair
 * stored at position t comes from the layer input x_t (it is the ephemeral
 * pair), so all positions are computed at once with causal attention. The
 * Figure 4 baseline. Excludes RT_FLAG_NAIVE_SCHEDULE. */
#define RT_FLAG_TRANSFORMER 4u
/* Query/key norm (translated paper section 2 notation, the separate RMS on
 * queries and keys after their projections; per head, as in the query/key
 * normalisation it cites): q, k' and the persistent k are each replaced by
 * g * x / sqrt(mean(x^2) + rms_eps) over each head's head_dim components,
 * with gains g_q (queries) and g_k (keys). bf16 layers: head_dim 32 or 64. */
#define RT_FLAG_QK_NORM 8u

/* Attention shape. softmax_scale (finite, >= 0) multiplies every score <k, q>
 * (the pages' operator has none, i.e. 1.0; workloads use 1/sqrt(head_dim)). */
typedef struct {
    int32_t batch, seq_len, n_heads, head_dim;
    rt_dtype dtype;
    float softmax_scale;
} rt_attn_desc;

/* Layer shape. d_model must equal n_heads*head_dim. rms_eps is the epsilon
 * of both RMS normalisations, RMS(v) = g * v / sqrt(mean(v^2) + eps).
 * residual_scale rho multiplies both residual branches (the pages use
 * 1/sqrt(number of layers); 1.0 gives the plain pre-LN layer).
 * kv_source_norm (0 or 1) chooses how an RT layer forms its persistent pair
 * from the output z_t (translated paper section 2.2, whose text breaks off
 * before this formula): 1 (the reading the workloads use) applies the same
 * map as the ephemeral pair, k_t = W_k RMS_attn(z_t), v_t = W_v RMS_attn(z_t);
 * 0 takes the formula literally, k_t = W_k z_t, v_t = W_v z_t (no RMS, no
 * g_attn). The Transformer layer (RT_FLAG_TRANSFORMER) needs 1: its pair is
 * its ephemeral pair. */
typedef struct {
    rt_attn_desc attn;
    int32_t d_model, d_ff;
    float rms_eps, residual_scale;
    int32_t kv_source_norm;
    uint32_t flags;
} rt_layer_desc;

/* Weights, device pointers in the descriptor's dtype, row-major [out][in]:
 * W_q, W_k, W_v, W_o: [d][d]; W_1: [F][d]; W_2: [d][F]. The same W_k, W_v
 * form the ephemeral pair (from x_t) and the persistent pair (from z_t).
 * g_attn (RMS gain before Q/K/V) and g_mlp (RMS gain before the MLP) are
 * fp32 [d], or NULL for a vector of ones; so are g_q and g_k, the query/key
 * norm gains (read only with RT_FLAG_QK_NORM; head h uses entries
 * h*head_dim .. h*head_dim+head_dim-1). A given g_attn or g_mlp is folded
 * into the projection it feeds, W[r][c] g[c], in fp32 (bf16 layers keep the
 * folded weight as two bf16 terms, the rounded product and its rounding
 * error, so the fold adds no bf16 rounding; those products then run over 2d
 * columns). */
typedef struct {
    const void *w_q, *w_k, *w_v, *w_o, *w_1, *w_2;
    const float *g_attn, *g_mlp;
    const float *g_q, *g_k;
} rt_layer_weights;

/*
 * rt_blocked_attn_update -- one step of the blocked schedule
 * (reading note, summary section 4.2): with b = largest power of two dividing
 * t, apply the persistent pairs of positions t-b+1..t to the online-softmax
 * state of queries t+1..min(t+b, N).
 *   q     [N][B][H][dh]  queries (dtype)
 *   k, v  [N][B][H][dh]  persistent keys / values; rows t-b+1..t are read
 *   m, l  [N][B][H]      fp32 state: running maximum of the base-2 logits
 *                        s = softmax_scale*log2(e)*<k,q>, and sum of 2^(s-m)
 *   o     [N][B][H][dh]  fp32 state: unnormalised numerator sum 2^(s-m) v
 * State row j (position j) is read and written only by steps that cover
 * query j. When t is a power of two the block starts at position 1, which
 * is the first step to touch any of its queries: the state of those rows is
 * then initialised, not read, so the caller never clears the state.
 * t must be in 1..N; t = N (no query left) is a valid no-op.
 */
rt_status rt_blocked_attn_update(const rt_attn_desc* desc, int32_t t,
                                 const void* q, const void* k, const void* v,
                                 float* m, float* l, float* o, rt_stream_t stream);

/*
 * rt_finalize_step -- attention output of position t: merge the ephemeral
 * pair (k'_t, v'_t) into query t's state and normalise, a_t = o / l
 * (translated paper section 2.2: the ephemeral pair is used only by position
 * t's own attention). At t = 1 the state is empty and a_1 = v'_1.
 *   q, k_eph, v_eph [N][B][H][dh] (dtype); rows t are read
 *   m, l [N][B][H], o [N][B][H][dh] (fp32): row t is read (not at t = 1), never written
 *   a_t [B][H*dh] (dtype): written
 * Call it after every update step t' < t has been enqueued.
 */
rt_status rt_finalize_step(const rt_attn_desc* desc, int32_t t,
                           const void* q, const void* k_eph, const void* v_eph,
                           const float* m, const float* l, const float* o,
                           void* a_t, rt_stream_t stream);

/*
 * rt_update_finalize_step -- step t of the blocked schedule fused with the
 * finalize of position t+1, in one launch: the pairs t-b+1..t are applied to
 * queries t+1..min(t+b, N) as rt_blocked_attn_update does, except that query
 * t+1, whose state is complete once step t is applied (every pair 1..t has
 * then reached it), is finished into a_next = attention output of position
 * t+1 (as rt_finalize_step(t+1) would) and its state row is not written.
 * This is the update a layer forward runs after each position.
 *   q, k_eph, v_eph, k, v [N][B][H][dh] (dtype); m, l [N][B][H], o [N][B][H][dh] (fp32)
 *   a_next [B][H*dh] (dtype): written
 * t must be in 1..N-1.
 */
rt_status rt_update_finalize_step(const rt_attn_desc* desc, int32_t t,
                                  const void* q, const void* k_eph, const void* v_eph,
                                  const void* k, const void* v,
                                  float* m, float* l, float* o, void* a_next, rt_stream_t stream);

/*
 * rt_attn_forward -- the blocked-schedule attention of a whole sequence with
 * every pair known up front (the update and finalize steps above, in order),
 * saving what its backward needs:
 *   q, k_eph, v_eph, k, v [N][B][H][dh] (dtype), read
 *   a   [N][B][H][dh] (dtype): attention outputs, written
 *   lse [N][B][H] fp32: each query's base-2 log-sum-exp, m + log2(l) in the
 *       state's units (s = softmax_scale*log2(e)*<k,q>), written
 *   m, l [N][B][H], o [N][B][H][dh] fp32: the online-softmax state (scratch)
 */
rt_status rt_attn_forward(const rt_attn_desc* desc, const void* q, const void* k_eph, const void* v_eph,
                          const void* k, const void* v, void* a, float* lse, float* m, float* l, float* o,
                          rt_stream_t stream);

/*
 * rt_attn_backward -- gradient of that attention for an output adjoint
 * a_bar = dL/da. The pages say only that the RT backward can be batched
 * outside the position loop (reading note, summary section 5.3; the
 * translated paper's backward section is missing); the gradient is the chain
 * rule through each query's softmax (D_t = <a_bar_t, a_t>, ds_i = p_i
 * (<a_bar_t, v_i> - D_t); v_bar_i += p_i a_bar_t, k_bar_i += sigma ds_i q_t,
 * q_bar_t += sigma ds_i k_i), applied in the forward's blocked rectangles
 * (step t: keys t-b+1..t against queries t+1..t+b) with probabilities
 * recomputed from the saved lse, plus one per-query pass for the ephemeral
 * pair.
 *   q, k_eph, v_eph, k, v, a [N][B][H][dh] (dtype), lse [N][B][H] fp32: as
 *       used and saved by rt_attn_forward
 *   a_bar [N][B][H][dh] fp32, read
 *   q_bar, k_eph_bar, v_eph_bar, k_bar, v_bar [N][B][H][dh] fp32: written
 *       (every element; the caller clears nothing)
 *   delta [N][B][H] fp32: scratch
 */
rt_status rt_attn_backward(const rt_attn_desc* desc, const void* q, const void* k_eph, const void* v_eph,
                           const void* k, const void* v, const void* a, const float* lse, const float* a_bar,
                           float* q_bar, float* k_eph_bar, float* v_eph_bar, float* k_bar, float* v_bar,
                           float* delta, rt_stream_t stream);

/*
 * rt_layer_workspace_bytes -- device workspace that rt_layer_forward and
 * rt_layer_plan_create need for this shape, or 0 for an invalid descriptor.
 */
size_t rt_layer_workspace_bytes(const rt_layer_desc* desc);

/*
 * rt_layer_forward -- the RT layer x -> z over positions 1..N for B
 * independent sequences (reading note, translated paper sections 2.1-2.2;
 * the unit timed in the paper's section 6 is this single-layer map):
 *   u_t = RMS_attn(x_t);  q_t, k'_t, v'_t = W_q u_t, W_k u_t, W_v u_t   (all t up front)
 *   a_t = per-head softmax attention of q_t over persistent pairs 1..t-1
 *         and the ephemeral pair t (blocked schedule)
 *   h_t = x_t + rho W_o a_t
 *   z_t = h_t + rho W_2 GELU(W_1 RMS_mlp(h_t))          (GELU with erf)
 *   k_t, v_t = W_k RMS_attn(z_t), W_v RMS_attn(z_t)      (persistent pair)
 *   x       [N][B][d]      input (dtype), read
 *   z       [N][B][d]      output (dtype), written
 *   k_cache [N][B][H][dh]  persistent keys (dtype), written: the KV cache a
 *   v_cache [N][B][H][dh]  later decode step would read
 *   workspace: device memory of at least rt_layer_workspace_bytes(desc),
 *              256-byte aligned; its contents are scratch.
 * The B sequences are independent (no exchange between batch rows).
 * desc->flags selects the schedule (blocked by default, RT_FLAG_NAIVE_SCHEDULE)
 * or the standard Transformer layer (RT_FLAG_TRANSFORMER); the workspace
 * size depends on that choice.
 */
rt_status rt_layer_forward(const rt_layer_desc* desc, const rt_layer_weights* w,
                           const void* x, void* z, void* k_cache, void* v_cache,
                           void* workspace, size_t workspace_bytes, rt_stream_t stream);

/*
 * Gradients of a layer's parameters, fp32, each shaped as its parameter:
 * w_q, w_k, w_v, w_o [d][d], w_1 [F][d], w_2 [d][F], g_attn, g_mlp [d].
 * The six weight gradients are required; a gain gradient may be NULL (then
 * it is not computed). Gains absent from rt_layer_weights are ones, and their
 * gradients are still defined.
 */
typedef struct {
    float *w_q, *w_k, *w_v, *w_o, *w_1, *w_2;
    float *g_attn, *g_mlp;
} rt_layer_grads;

/*
 * rt_layer_backward_workspace_bytes -- device workspace of rt_layer_backward,
 * or 0 for an invalid or unsupported descriptor.
 */
size_t rt_layer_backward_workspace_bytes(const rt_layer_desc* desc);

/*
 * rt_layer_backward -- gradient of L = sum(z_bar * z) for the RT layer map of
 * rt_layer_forward. The pages give the backward only as an idea: it can be
 * batched outside the position loop, with the persistent pairs rebuilt from
 * the stored outputs (translated paper section 6.1; section 6.4 is a heading
 * without a body). The gradient here is the chain rule:
 *   - recompute, batched over all N*B rows: q, k', v' from x; the persistent
 *     k, v from the given z; the blocked attention with each query's
 *     log-sum-exp; h; the MLP's pre-activation u;
 *   - positions in reverse: step t's attention rectangle (its queries are all
 *     differentiated by then, so row t's k_bar, v_bar are complete), then
 *       z_bar_t += RMS_attn'(z_t)^T (W_k^T k_bar_t + W_v^T v_bar_t)
 *       u_bar = rho (W_2^T z_bar_t) * GELU'(u_t)
 *       h_bar = z_bar_t + RMS_mlp'(h_t)^T (W_1^T u_bar);  a_bar_t = rho W_o^T h_bar
 *     and query t's own pass (D_t, the ephemeral pair, q_bar's first term);
 *   - batched again: x_bar = h_bar + RMS_attn'(x)^T (W_q^T q_bar + W_k^T k'_bar
 *     + W_v^T v'_bar), every weight gradient as a sum over positions and rows
 *     of (adjoint of a product's output) x (its input), the gains' gradients.
 *   x      [N][B][d] (dtype): the forward's input, read
 *   z      [N][B][d] (dtype): the forward's output as stored, read
 *   z_bar  [N][B][d] fp32: the output adjoint, read
 *   x_bar  [N][B][d] fp32: the input adjoint, written
 *   grads: written (overwritten, not accumulated)
 *   workspace: at least rt_layer_backward_workspace_bytes(desc), 256-byte aligned.
 * bf16 layers keep adjoints in fp32; a product reads them rounded to bf16 and
 * accumulates in fp32. Roundings of the forward's stored values are taken as
 * the identity (their derivative is not defined). Supported: the RT layer
 * with the blocked or naive schedule (the same map); not RT_FLAG_TRANSFORMER
 * or RT_FLAG_QK_NORM (RT_ERR_UNSUPPORTED).
 */
rt_status rt_layer_backward(const rt_layer_desc* desc, const rt_layer_weights* w, const void* x, const void* z,
                            const float* z_bar, float* x_bar, const rt_layer_grads* grads,
                            void* workspace, size_t workspace_bytes, rt_stream_t stream);

/*
 * rt_layer_decode_workspace_bytes -- device workspace of rt_layer_decode_step
 * (independent of seq_len and n_past), or 0 for an invalid descriptor.
 */
size_t rt_layer_decode_workspace_bytes(const rt_layer_desc* desc);

/*
 * rt_layer_decode_step -- autoregressive decoding of one new position
 * t = n_past + 1 per sequence against the persistent KV cache a prefill (or
 * earlier decode steps) left behind (translated paper section 7.3: each new
 * token attends to keys and values cached from the earlier tokens, the same
 * per-token work as a Transformer's decode). The layer map of one position
 * of rt_layer_forward:
 *   q, k', v' from x_t; a_t = attention over cached pairs 1..n_past and (k'_t, v'_t);
 *   z_t = the layer's output; the persistent pair (k_t, v_t) from z_t is
 *   appended at row n_past of the caches (with RT_FLAG_TRANSFORMER: (k'_t, v'_t)).
 *   desc->attn.seq_len: the caches' capacity in positions; 0 <= n_past < seq_len
 *   x_t     [B][d]          input of the new position (dtype), read
 *   z_t     [B][d]          output (dtype), written
 *   k_cache [seq_len][B][H][dh], v_cache likewise (dtype): rows 0..n_past-1
 *           read, row n_past written, later rows untouched
 *   workspace: at least rt_layer_decode_workspace_bytes(desc), 256-byte aligned.
 * n_past = 0 is the first position (a_1 = v'_1). RT_FLAG_NAIVE_SCHEDULE has
 * no effect here (one position has one schedule).
 */
rt_status rt_layer_decode_step(const rt_layer_desc* desc, const rt_layer_weights* w, int32_t n_past,
                               const void* x_t, void* z_t, void* k_cache, void* v_cache,
                               void* workspace, size_t workspace_bytes, rt_stream_t stream);

/*
 * rt_layer_decode_step_static -- rt_layer_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same computation and kernels, with no
 * workspace argument. Its scratch is a device array of
 * RT_DECODE_STATIC_SCRATCH_BYTES inside the library; every GPU that loads the
 * library holds its own copy until the process ends. The call allocates
 * nothing (no hipMalloc, no allocating library routine).
 *   Arguments, layouts and results: as rt_layer_decode_step.
 *   RT_ERR_WORKSPACE when rt_layer_decode_workspace_bytes(desc) exceeds
 *   RT_DECODE_STATIC_SCRATCH_BYTES (e.g. B=512, d=1024, F=4096 with RMS
 *   gains needs ~39 MiB: it fits).
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents (nothing in it needs clearing: every byte a call reads, the same
 * call has written). Calls that overlap in time on one GPU (two streams, two
 * host threads) race on the array: serialise them.
 */
#define RT_DECODE_STATIC_SCRATCH_BYTES (64u << 20)
rt_status rt_layer_decode_step_static(const rt_layer_desc* desc, const rt_layer_weights* w, int32_t n_past,
                                      const void* x_t, void* z_t, void* k_cache, void* v_cache,
                                      rt_stream_t stream);

/*
 * Plans: the same computation as rt_layer_forward, with its O(N) launches
 * recorded once into a HIP graph and replayed by one launch (the paper's
 * section 6.2 records its step loop as a CUDA graph for the same reason).
 * The pointers given at creation are baked into the graph: the buffers must
 * stay allocated, and keep their meaning, until rt_layer_plan_destroy.
 * A plan may be launched any number of times, on any stream.
 */
typedef struct rt_plan rt_plan;
rt_status rt_layer_plan_create(const rt_layer_desc* desc, const rt_layer_weights* w,
                               const void* x, void* z, void* k_cache, void* v_cache,
                               void* workspace, size_t workspace_bytes, rt_plan** plan);
rt_status rt_layer_plan_launch(rt_plan* plan, rt_stream_t stream);
void rt_layer_plan_destroy(rt_plan* plan);

/*
 * Stacks: n_layers RT layers of one shape, layer l's input being layer
 * l-1's output (translated paper section 6.1: each layer's stored output z
 * is the next layer's input), so x -> z[n_layers-1] is the model's forward.
 *   desc      one descriptor for every layer (shape, dtype, flags)
 *   w         [n_layers] the layers' weights
 *   x         [N][B][d] input of layer 0 (dtype), read
 *   z         [n_layers] outputs [N][B][d] (dtype), written; z[l] is layer l+1's input
 *   k_cache, v_cache  [n_layers] persistent pairs [N][B][H][dh] of each layer, written
 *   workspace: at least rt_stack_workspace_bytes(desc, n_layers), 256-byte aligned.
 * Each layer computes the map of rt_layer_forward, with the same schedule.
 * Blocked layers run as a wavefront: layer l works on position t while layer
 * l-1 is C + 8 positions ahead (C = the power of two N/16 rounded down, at
 * least 8), and the per-position products of all layers share one launch
 * each. Each layer after the first projects its queries and ephemeral pairs
 * in chunks of C positions as its input becomes available; a blocked step
 * whose block reaches queries not yet projected applies it to them when
 * their chunk is, before any later step, so every query merges the same
 * blocks in the same order as layer by layer. The naive schedule and the
 * Transformer layer run layer after layer. Buffers must not overlap.
 * n_layers: 1..1024.
 */
size_t rt_stack_workspace_bytes(const rt_layer_desc* desc, int32_t n_layers);
rt_status rt_stack_forward(const rt_layer_desc* desc, int32_t n_layers, const rt_layer_weights* w,
                           const void* x, void* const* z, void* const* k_cache, void* const* v_cache,
                           void* workspace, size_t workspace_bytes, rt_stream_t stream);
/* The stack's launches recorded as one HIP graph (launch and destroy it as a
 * layer plan; the same lifetime rules). */
rt_status rt_stack_plan_create(const rt_layer_desc* desc, int32_t n_layers, const rt_layer_weights* w,
                               const void* x, void* const* z, void* const* k_cache, void* const* v_cache,
                               void* workspace, size_t workspace_bytes, rt_plan** plan);

/*
 * rt_schedule_step -- the integer rule of the blocked schedule on the host
 * (reading note, summary section 4.2): for step t of an N-position sequence,
 * the KV block [*kv_first, *kv_last] and the query block
 * [*q_first, *q_last] (1-based, inclusive; empty when *q_first > *q_last).
 * No HIP call.
 */
rt_status rt_schedule_step(int32_t t, int32_t n, int32_t* kv_first, int32_t* kv_last,
                           int32_t* q_first, int32_t* q_last);

/* Text of the calling thread's last error ("" if none). Never NULL. */
const char* rt_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RT_PREFILL_H */
