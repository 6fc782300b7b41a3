// Blocked-schedule attention update and finalize kernels.
//
// Recurrent Transformer reading note (lshu.cn/news/403416), summary section
// 4.2: each query keeps an online-softmax state (running maximum m,
// normaliser l, numerator o); a step merges a block of persistent key/value
// pairs into the states of a block of queries. The per-block merge is the
// tile merge of IO-aware exact attention (FlashAttention paragraph of the
// long-context survey translation, blog.csdn.net/yorkhunter/article/details/138851205).
// Scores are kept in base 2: s = softmax_scale * log2(e) * <k, q>, so the
// exponentials are the hardware exp2.
#include "rt_device.h"
#include "rt_internal.h"

namespace rt {

// SIMT update: one item = (query row i, batch*head pair p), handled by a
// group of DH/8 consecutive lanes, each holding 8 of the DH components.
// Items are ordered pair-fastest, so neighbouring groups read neighbouring
// 16-byte pieces of the position-major q / k / v / state slabs.
template <typename T, int DH>
__global__ __launch_bounds__(256) void update_simt_kernel(UpdateArgs a) {
    constexpr int G = DH / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t item = gid / G;
    const int lane = (int)(gid % G);
    if (item >= (int64_t)a.nq * a.P) return;  // whole groups leave together
    const int64_t i = item / a.P;
    const int64_t p = item % a.P;
    const int64_t j = a.q0 + i;
    const int64_t slab = a.P * DH;  // elements per position
    const int64_t off = p * DH + lane * 8;

    float qv[8];
    load8((const T*)a.q + j * slab + off, qv);
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] *= a.sigma2;

    // the block's own softmax partial
    float mb = -INFINITY, lb = 0.f, ob[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const T* kp = (const T*)a.k + (int64_t)a.kv0 * slab + off;
    const T* vp = (const T*)a.v + (int64_t)a.kv0 * slab + off;
    for (int s = 0; s < a.nkv; ++s) {
        float kv[8], vv[8];
        load8(kp + s * slab, kv);
        load8(vp + s * slab, vv);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += qv[e] * kv[e];
        d = group_sum<G>(d);
        const float mn = fmaxf(mb, d);
        const float c = fast_exp2(mb - mn);
        const float pe = fast_exp2(d - mn);
        lb = lb * c + pe;
#pragma unroll
        for (int e = 0; e < 8; ++e) ob[e] = ob[e] * c + pe * vv[e];
        mb = mn;
    }

    // merge with the stored state of this query
    const int64_t sidx = j * a.P + p;
    if (!a.init) {
        const float ms = a.m[sidx], ls = a.l[sidx];
        float os[8];
        load8(a.o + sidx * DH + lane * 8, os);
        const float mn = fmaxf(ms, mb);
        const float cs = fast_exp2(ms - mn), cb = fast_exp2(mb - mn);
        lb = ls * cs + lb * cb;
#pragma unroll
        for (int e = 0; e < 8; ++e) ob[e] = os[e] * cs + ob[e] * cb;
        mb = mn;
    }

    if (a.fin && i == 0) {
        // the ephemeral pair of this position, then a = o / l
        float ke[8], ve[8];
        load8((const T*)a.k_eph + j * slab + off, ke);
        load8((const T*)a.v_eph + j * slab + off, ve);
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) d += qv[e] * ke[e];
        d = group_sum<G>(d);
        const float mn = fmaxf(mb, d);
        const float c = fast_exp2(mb - mn);
        const float pe = fast_exp2(d - mn);
        lb = lb * c + pe;
        const float inv = 1.0f / lb;
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = (ob[e] * c + pe * ve[e]) * inv;
        store8((T*)a.a_out + off, out);
    } else {
        if (lane == 0) {
            a.m[sidx] = mb;
            a.l[sidx] = lb;
        }
        store8(a.o + sidx * DH + lane * 8, ob);
    }
}

template <typename T, int DH>
static hipError_t launch_simt(const UpdateArgs& a, hipStream_t s) {
    const int64_t threads = (int64_t)a.nq * a.P * (DH / 8);
    if (threads <= 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((update_simt_kernel<T, DH>), dim3((uint32_t)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_typed(int head_dim, const UpdateArgs& a, hipStream_t s) {
    switch (head_dim) {
        case 32: return launch_simt<T, 32>(a, s);
        case 64: return launch_simt<T, 64>(a, s);
        case 128: return launch_simt<T, 128>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_update(rt_dtype dt, int head_dim, const UpdateArgs& a, hipStream_t s) {
    return dt == RT_BF16 ? launch_typed<bf16>(head_dim, a, s) : launch_typed<float>(head_dim, a, s);
}

}  // namespace rt
