// Backward of the RT attention map under the blocked schedule.
//
// The pages say only that the RT backward can be batched outside the
// position loop (Recurrent Transformer reading note, summary section 5.3;
// translated paper section 6.4, whose body is missing). Here the gradient of
// the attention map is derived per query t (scores s_i = sigma <q_t, k_i>,
// softmax p, output a_t; D_t = <a_bar_t, a_t>, ds_i = p_i (<a_bar_t, v_i> - D_t)):
//   v_bar_i += p_i a_bar_t,  k_bar_i += sigma ds_i q_t,  q_bar_t += sigma ds_i k_i,
// and applied in the same rectangles as the forward: step t pairs the block
// of keys (t-b, t] with the queries (t, t+b], so every (key, query) pair of
// the causal triangle is visited once and the probabilities are recomputed
// from the query's saved log-sum-exp (base 2, as the forward keeps its
// logits). The ephemeral pair of each query is a separate per-query pass.
#include "rt_device.h"
#include "rt_internal.h"

namespace rt {

// One 8-lane group per (query j, pair p), items pair-fastest: delta_j, and the
// query's own ephemeral pair (its only reader): k'_bar, v'_bar and q_bar's
// first term, written (not accumulated).
template <typename T, int DH>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BackwardArgs b) {
    constexpr int G = DH / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t item = gid / G;
    const int lane = (int)(gid % G);
    if (item >= (int64_t)b.n_pos * b.P) return;
    const int64_t j = item / b.P, p = item % b.P;
    const int64_t off = (j * b.P + p) * DH + lane * 8;
    float q[8], ke[8], ve[8], a[8], ab[8];
    load8((const T*)b.q + off, q);
    load8((const T*)b.k_eph + off, ke);
    load8((const T*)b.v_eph + off, ve);
    load8((const T*)b.a + off, a);
    load8(b.a_bar + off, ab);
    float dd = 0.f, se = 0.f, dpe = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        dd += ab[e] * a[e];
        se += q[e] * ke[e];
        dpe += ab[e] * ve[e];
    }
    dd = group_sum<G>(dd);
    se = group_sum<G>(se);
    dpe = group_sum<G>(dpe);
    const float pe = fast_exp2(se * b.sigma2 - b.lse[j * b.P + p]);
    const float ds = pe * (dpe - dd);
    float kb[8], vb[8], qb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        kb[e] = b.sigma * ds * q[e];
        vb[e] = pe * ab[e];
        qb[e] = b.sigma * ds * ke[e];
    }
    store8(b.k_eph_bar + off, kb);
    store8(b.v_eph_bar + off, vb);
    store8(b.q_bar + off, qb);
    if (lane == 0) b.delta[j * b.P + p] = dd;
}

// Step rectangle, key side: one 8-lane group per (key row i, pair p) loops over
// the step's queries. The block's last row is first touched by this step (a
// row's first step is its own position), so it is set; the others accumulate.
template <typename T, int DH>
__global__ __launch_bounds__(256) void bwd_kv_kernel(BackwardArgs b, int32_t kv0, int32_t nkv, int32_t q0, int32_t nq) {
    constexpr int G = DH / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t item = gid / G;
    const int lane = (int)(gid % G);
    if (item >= (int64_t)nkv * b.P) return;
    const int64_t i = kv0 + item / b.P, p = item % b.P;
    const int64_t slab = b.P * DH, off = p * DH + lane * 8;
    float k[8], v[8];
    load8((const T*)b.k + i * slab + off, k);
    load8((const T*)b.v + i * slab + off, v);
    float kb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, vb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int jj = 0; jj < nq; ++jj) {
        const int64_t j = q0 + jj;
        float q[8], ab[8];
        load8((const T*)b.q + j * slab + off, q);
        load8(b.a_bar + j * slab + off, ab);
        const float lse = b.lse[j * b.P + p], dd = b.delta[j * b.P + p];
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s += q[e] * k[e];
            dp += ab[e] * v[e];
        }
        s = group_sum<G>(s);
        dp = group_sum<G>(dp);
        const float pr = fast_exp2(s * b.sigma2 - lse);
        const float ds = pr * (dp - dd);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kb[e] += b.sigma * ds * q[e];
            vb[e] += pr * ab[e];
        }
    }
    float* kr = b.k_bar + i * slab + off;
    float* vr = b.v_bar + i * slab + off;
    if (i != kv0 + nkv - 1) {
        float ko[8], vo[8];
        load8(kr, ko);
        load8(vr, vo);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kb[e] += ko[e];
            vb[e] += vo[e];
        }
    }
    store8(kr, kb);
    store8(vr, vb);
}

// Step rectangle, query side: one 8-lane group per (query row j, pair p) loops
// over the step's keys and adds its term to q_bar_j.
template <typename T, int DH>
__global__ __launch_bounds__(256) void bwd_q_kernel(BackwardArgs b, int32_t kv0, int32_t nkv, int32_t q0, int32_t nq) {
    constexpr int G = DH / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t item = gid / G;
    const int lane = (int)(gid % G);
    if (item >= (int64_t)nq * b.P) return;
    const int64_t j = q0 + item / b.P, p = item % b.P;
    const int64_t slab = b.P * DH, off = p * DH + lane * 8;
    float q[8], ab[8];
    load8((const T*)b.q + j * slab + off, q);
    load8(b.a_bar + j * slab + off, ab);
    const float lse = b.lse[j * b.P + p], dd = b.delta[j * b.P + p];
    float qb[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int ii = 0; ii < nkv; ++ii) {
        const int64_t i = kv0 + ii;
        float k[8], v[8];
        load8((const T*)b.k + i * slab + off, k);
        load8((const T*)b.v + i * slab + off, v);
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s += q[e] * k[e];
            dp += ab[e] * v[e];
        }
        s = group_sum<G>(s);
        dp = group_sum<G>(dp);
        const float ds = fast_exp2(s * b.sigma2 - lse) * (dp - dd);
#pragma unroll
        for (int e = 0; e < 8; ++e) qb[e] += b.sigma * ds * k[e];
    }
    float* qr = b.q_bar + j * slab + off;
    float qo[8];
    load8(qr, qo);
#pragma unroll
    for (int e = 0; e < 8; ++e) qb[e] += qo[e];
    store8(qr, qb);
}

__global__ __launch_bounds__(256) void bwd_zero_kernel(float* x, float* y, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        x[i] = 0.f;
        y[i] = 0.f;
    }
}

static dim3 grid_for(int64_t items, int DH) { return dim3((uint32_t)((items * (DH / 8) + 255) / 256)); }

template <typename T>
static hipError_t prep_typed(int dh, const BackwardArgs& b, hipStream_t s) {
    const int64_t items = (int64_t)b.n_pos * b.P;
    switch (dh) {
        case 32: hipLaunchKernelGGL((bwd_prep_kernel<T, 32>), grid_for(items, 32), dim3(256), 0, s, b); break;
        case 64: hipLaunchKernelGGL((bwd_prep_kernel<T, 64>), grid_for(items, 64), dim3(256), 0, s, b); break;
        case 128: hipLaunchKernelGGL((bwd_prep_kernel<T, 128>), grid_for(items, 128), dim3(256), 0, s, b); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, int DH>
static hipError_t step_dh(const BackwardArgs& b, int32_t kv0, int32_t nkv, int32_t q0, int32_t nq, hipStream_t s) {
    hipLaunchKernelGGL((bwd_kv_kernel<T, DH>), grid_for((int64_t)nkv * b.P, DH), dim3(256), 0, s, b, kv0, nkv, q0, nq);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_q_kernel<T, DH>), grid_for((int64_t)nq * b.P, DH), dim3(256), 0, s, b, kv0, nkv, q0, nq);
    return hipGetLastError();
}

template <typename T>
static hipError_t step_typed(int dh, const BackwardArgs& b, int32_t kv0, int32_t nkv, int32_t q0, int32_t nq,
                             hipStream_t s) {
    switch (dh) {
        case 32: return step_dh<T, 32>(b, kv0, nkv, q0, nq, s);
        case 64: return step_dh<T, 64>(b, kv0, nkv, q0, nq, s);
        case 128: return step_dh<T, 128>(b, kv0, nkv, q0, nq, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_backward_prep(rt_dtype dt, int head_dim, const BackwardArgs& b, hipStream_t s) {
    if (b.n_pos <= 0) return hipSuccess;
    return dt == RT_BF16 ? prep_typed<bf16>(head_dim, b, s) : prep_typed<float>(head_dim, b, s);
}

hipError_t launch_backward_step(rt_dtype dt, int head_dim, const BackwardArgs& b, int32_t kv0, int32_t nkv,
                                int32_t q0, int32_t nq, hipStream_t s) {
    if (nkv <= 0 || nq <= 0) return hipSuccess;
    return dt == RT_BF16 ? step_typed<bf16>(head_dim, b, kv0, nkv, q0, nq, s)
                         : step_typed<float>(head_dim, b, kv0, nkv, q0, nq, s);
}

hipError_t launch_backward_zero_rows(int head_dim, const BackwardArgs& b, int32_t row0, int32_t rows,
                                     hipStream_t s) {
    const int64_t n = (int64_t)rows * b.P * head_dim;
    if (n <= 0) return hipSuccess;
    const int64_t off = (int64_t)row0 * b.P * head_dim;
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, b.k_bar + off,
                       b.v_bar + off, n);
    return hipGetLastError();
}

}  // namespace rt
