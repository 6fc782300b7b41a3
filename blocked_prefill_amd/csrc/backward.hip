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

// Workgroup barrier ordering LDS accesses only.
__device__ __forceinline__ void lds_fence_barrier_bwd() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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
__device__ __forceinline__ void bwd_kv_item(const BackwardArgs& b, int64_t item, int lane, int32_t kv0, int32_t nkv,
                                            int32_t q0, int32_t nq) {
    constexpr int G = DH / 8;
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
    if (b.kv_accumulate || i != kv0 + nkv - 1) {
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
__device__ __forceinline__ void bwd_q_item(const BackwardArgs& b, int64_t item, int lane, int32_t kv0, int32_t nkv,
                                           int32_t q0, int32_t nq) {
    constexpr int G = DH / 8;
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

// Both sides of a step in one launch: items [0, nkv*P) are keys, the rest
// queries. A wave may hold both kinds, but each G-lane group is one item, so
// the group sums' shuffles never cross from one kind to the other.
template <typename T, int DH>
__global__ __launch_bounds__(256) void bwd_step_kernel(BackwardArgs b, int32_t kv0, int32_t nkv, int32_t q0,
                                                        int32_t nq) {
    constexpr int G = DH / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t item = gid / G;
    const int lane = (int)(gid % G);
    const int64_t nk_items = (int64_t)nkv * b.P;
    if (item < nk_items)
        bwd_kv_item<T, DH>(b, item, lane, kv0, nkv, q0, nq);
    else if (item < nk_items + (int64_t)nq * b.P)
        bwd_q_item<T, DH>(b, item - nk_items, lane, kv0, nkv, q0, nq);
}

// ---------------------------------------------------------------- MFMA (bf16, head_dim 64, blocks >= 32)
//
// Same layout facts as the forward's MFMA update (v_mfma_f32_32x32x16_bf16:
// A lane l holds row l%32, k (l/32)*8..+8; B lane l holds column l%32, k
// (l/32)*8..+8; C element e of lane l is row 8(e/4) + 4(l/32) + e%4, column
// l%32). Feeding the A rows with bits 2 and 3 of the row index swapped makes
// the 16 results a lane holds for its column cover rows (e&7) + 8(l/32) +
// 16(e>>3): exactly the B-operand layout of a following product, so
// probabilities and score gradients never leave registers.

__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Item of workgroup i when the grid divides by 8: XCD i % 8 gets items
// (i % 8) * (grid / 8) + 0, 1, ... in dispatch order (a contiguous range of pairs).
__device__ __forceinline__ int64_t xcd_item(int64_t i, int64_t grid) {
    return (grid & 7) == 0 ? (i & 7) * (grid >> 3) + (i >> 3) : i;
}

// Query side: a wave owns 32 queries (columns). Per chunk of 32 keys:
//   S^T = K Q^T, dP^T = V a_bar^T (A = K, V rows in LDS; B = this wave's q, a_bar)
//   P^T = 2^(sigma2 S^T - lse), dS^T = P^T (dP^T - delta)
//   dQ^T += K^T dS^T                (A = K^T in LDS)
// and q_bar += sigma dQ at the end.
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void bwd_q_mfma_kernel(BackwardArgs b, int32_t kv0, int32_t nkv, int32_t q0,
                                                                 int32_t nq, int nqt) {
    constexpr int DH = 64, KT = 64, STR = 72, NT = 64 * WAVES;
    __shared__ __attribute__((aligned(16))) bf16 Ks[KT * STR];
    __shared__ __attribute__((aligned(16))) bf16 Vs[KT * STR];
    __shared__ __attribute__((aligned(16))) bf16 Kt[DH * STR];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, ql = lane & 31;
    // each XCD (workgroup i runs on XCD i % 8) takes a contiguous range of (pair, tile) items
    const int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int64_t pair = item / nqt;
    const int qtile = (int)(item % nqt);
    const int64_t slab = b.P * DH;
    const int wq0 = qtile * 32 * WAVES + wave * 32;
    const bool active = wq0 < nq;
    const int qrow = wq0 + ql;
    const bool qvalid = qrow < nq;
    const int64_t j = (int64_t)q0 + min(qrow, nq - 1);
    // a_bar enters dP as two bf16 terms (the rounded value and its rounding
    // error): dS = P (dP - delta) subtracts dP's weighted mean, so dP's relative
    // rounding error would be amplified in dS
    bf16x8 qop[4], aop[4], alo[4];
    {
        const bf16* qp = (const bf16*)b.q + j * slab + pair * DH + 8 * g;
        const float* ap = b.a_bar + j * slab + pair * DH + 8 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qop[i] = *reinterpret_cast<const bf16x8*>(qp + 16 * i);
            const float4 x0 = *reinterpret_cast<const float4*>(ap + 16 * i);
            const float4 x1 = *reinterpret_cast<const float4*>(ap + 16 * i + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                aop[i][e] = (bf16)xs[e];
                alo[i][e] = (bf16)(xs[e] - (float)aop[i][e]);
            }
        }
    }
    // a query past the block weighs 0: lse = +inf makes its probabilities 0
    const float lse = qvalid ? b.lse[j * b.P + pair] : INFINITY;
    const float dd = b.delta[j * b.P + pair];
    const float sigma2 = b.sigma2;
    f32x16 d0, d1;  // dQ^T, dh 0..31 and 32..63
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        d0[e] = 0.f;
        d1[e] = 0.f;
    }
    const bf16* kb = (const bf16*)b.k + (int64_t)kv0 * slab + pair * DH;
    const bf16* vb = (const bf16*)b.v + (int64_t)kv0 * slab + pair * DH;
    const int krow = swap23(ql);
    for (int kt0 = 0; kt0 < nkv; kt0 += KT) {
        const int rows = min(nkv - kt0, KT);  // the last tile may be short (a block of 16)
        lds_fence_barrier_bwd();
        for (int c = tid; c < KT * 8; c += NT) {
            const int r = min(c >> 3, rows - 1), ch = (c & 7) * 8;
            const bf16x8 kx = *reinterpret_cast<const bf16x8*>(kb + (int64_t)(kt0 + r) * slab + ch);
            const bf16x8 vx = *reinterpret_cast<const bf16x8*>(vb + (int64_t)(kt0 + r) * slab + ch);
            *reinterpret_cast<bf16x8*>(&Ks[(c >> 3) * STR + ch]) = kx;
            *reinterpret_cast<bf16x8*>(&Vs[(c >> 3) * STR + ch]) = vx;
#pragma unroll
            for (int e = 0; e < 8; ++e) Kt[(ch + e) * STR + (c >> 3)] = kx[e];
        }
        lds_fence_barrier_bwd();
        if (!active) continue;
        for (int c32 = 0; c32 < rows; c32 += 32) {
            f32x16 st, dp;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                st[e] = 0.f;
                dp[e] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[(c32 + krow) * STR + 16 * i + 8 * g]);
                const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[(c32 + krow) * STR + 16 * i + 8 * g]);
                st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[i], st, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, alo[i], dp, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, aop[i], dp, 0, 0, 0);
            }
            // dS^T in the B layout: keys 8g.. (e < 8) and 16+8g.. (e >= 8), as two bf16
            // terms each (the rounded value and its rounding error): a query's score
            // gradients sum to zero, so q_bar = sigma sum_i dS_i k_i cancels, and one
            // bf16 rounding of dS would leave ~1e-2 relative error in it
            bf16x8 s0, s1, r0, r1;
            // keys past a short block's end repeat its last row: their score gradients are zeroed
            const int live = rows - c32 - 8 * g;  // keys 8g + e (e < live) and 16 + 8g + e (e < live - 16) exist
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pa = fast_exp2(__builtin_fmaf(st[e], sigma2, -lse));
                const float pb = fast_exp2(__builtin_fmaf(st[e + 8], sigma2, -lse));
                const float da = e < live ? pa * (dp[e] - dd) : 0.f;
                const float db = e + 16 < live ? pb * (dp[e + 8] - dd) : 0.f;
                s0[e] = (bf16)da;
                s1[e] = (bf16)db;
                r0[e] = (bf16)(da - (float)s0[e]);
                r1[e] = (bf16)(db - (float)s1[e]);
            }
            const bf16x8 klo0 = *reinterpret_cast<const bf16x8*>(&Kt[ql * STR + c32 + 8 * g]);
            const bf16x8 klo1 = *reinterpret_cast<const bf16x8*>(&Kt[ql * STR + c32 + 8 * g + 16]);
            const bf16x8 khi0 = *reinterpret_cast<const bf16x8*>(&Kt[(32 + ql) * STR + c32 + 8 * g]);
            const bf16x8 khi1 = *reinterpret_cast<const bf16x8*>(&Kt[(32 + ql) * STR + c32 + 8 * g + 16]);
            d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo0, r0, d0, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo1, r1, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi0, r0, d1, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi1, r1, d1, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo0, s0, d0, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo1, s1, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi0, s0, d1, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi1, s1, d1, 0, 0, 0);
        }
    }
    if (!qvalid) return;
    // this lane holds dh = blk*32 + 8*ee + 4*g + (0..3) of its query
    float* qr = b.q_bar + j * slab + pair * DH;
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
        float4* p0 = reinterpret_cast<float4*>(qr + 8 * ee + 4 * g);
        float4* p1 = reinterpret_cast<float4*>(qr + 32 + 8 * ee + 4 * g);
        float4 x0 = *p0, x1 = *p1;
        x0.x += b.sigma * d0[4 * ee + 0]; x0.y += b.sigma * d0[4 * ee + 1];
        x0.z += b.sigma * d0[4 * ee + 2]; x0.w += b.sigma * d0[4 * ee + 3];
        x1.x += b.sigma * d1[4 * ee + 0]; x1.y += b.sigma * d1[4 * ee + 1];
        x1.z += b.sigma * d1[4 * ee + 2]; x1.w += b.sigma * d1[4 * ee + 3];
        *p0 = x0;
        *p1 = x1;
    }
}

// Key side: a wave owns 32 keys (columns). Per chunk of 32 queries:
//   S = Q K^T, dP = a_bar V^T   (A = q, a_bar rows in LDS; B = this wave's k, v)
//   P = 2^(sigma2 S - lse), dS = P (dP - delta)   (lse, delta per query row, from LDS)
//   dV^T += a_bar^T P,  dK^T += Q^T dS            (A = transposed rows in LDS)
// and k_bar, v_bar rows written at the end (set on the block's last row, which
// this step touches first; accumulated elsewhere).
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void bwd_kv_mfma_kernel(BackwardArgs b, int32_t kv0, int32_t nkv, int32_t q0,
                                                                  int32_t nq, int nkt) {
    constexpr int DH = 64, QT = 64, STR = 72, NT = 64 * WAVES;
    __shared__ __attribute__((aligned(16))) bf16 Qs[QT * STR];
    __shared__ __attribute__((aligned(16))) bf16 As[QT * STR];
    __shared__ __attribute__((aligned(16))) bf16 Al[QT * STR];  // a_bar's rounding error (dP, as on the query side)
    __shared__ __attribute__((aligned(16))) bf16 Qt[DH * STR];
    __shared__ __attribute__((aligned(16))) bf16 At[DH * STR];
    __shared__ __attribute__((aligned(16))) float Ls[QT];
    __shared__ __attribute__((aligned(16))) float Ds[QT];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, kl = lane & 31;
    const int64_t item = xcd_item(blockIdx.x, gridDim.x);
    const int64_t pair = item / nkt;
    const int ktile = (int)(item % nkt);
    const int64_t slab = b.P * DH;
    const int wk0 = ktile * 32 * WAVES + wave * 32;
    const bool active = wk0 < nkv;
    const int krow_local = wk0 + kl;
    const bool kvalid = krow_local < nkv;
    const int64_t i_row = (int64_t)kv0 + min(krow_local, nkv - 1);
    bf16x8 kop[4], vop[4];
    {
        const bf16* kp = (const bf16*)b.k + i_row * slab + pair * DH + 8 * g;
        const bf16* vp = (const bf16*)b.v + i_row * slab + pair * DH + 8 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kop[i] = *reinterpret_cast<const bf16x8*>(kp + 16 * i);
            vop[i] = *reinterpret_cast<const bf16x8*>(vp + 16 * i);
        }
    }
    const float sigma2 = b.sigma2;
    f32x16 dv0, dv1, dk0, dk1;  // dV^T and dK^T, dh 0..31 and 32..63
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        dv0[e] = 0.f;
        dv1[e] = 0.f;
        dk0[e] = 0.f;
        dk1[e] = 0.f;
    }
    const bf16* qb = (const bf16*)b.q + (int64_t)q0 * slab + pair * DH;
    const float* ab = b.a_bar + (int64_t)q0 * slab + pair * DH;
    const int arow = swap23(kl);
    for (int qt0 = 0; qt0 < nq; qt0 += QT) {
        const int rows = min(nq - qt0, QT);
        lds_fence_barrier_bwd();
        for (int c = tid; c < QT * 8; c += NT) {
            const int r = min(c >> 3, rows - 1), ch = (c & 7) * 8;
            const bf16x8 qx = *reinterpret_cast<const bf16x8*>(qb + (int64_t)(qt0 + r) * slab + ch);
            const float4 a0 = *reinterpret_cast<const float4*>(ab + (int64_t)(qt0 + r) * slab + ch);
            const float4 a1 = *reinterpret_cast<const float4*>(ab + (int64_t)(qt0 + r) * slab + ch + 4);
            const float as_[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            bf16x8 ax, al;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ax[e] = (bf16)as_[e];
                al[e] = (bf16)(as_[e] - (float)ax[e]);
            }
            *reinterpret_cast<bf16x8*>(&Qs[(c >> 3) * STR + ch]) = qx;
            *reinterpret_cast<bf16x8*>(&As[(c >> 3) * STR + ch]) = ax;
            *reinterpret_cast<bf16x8*>(&Al[(c >> 3) * STR + ch]) = al;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                Qt[(ch + e) * STR + (c >> 3)] = qx[e];
                At[(ch + e) * STR + (c >> 3)] = ax[e];
            }
        }
        for (int r = tid; r < QT; r += NT) {
            // queries past the block weigh 0 (lse = +inf)
            const int64_t jq = (int64_t)q0 + qt0 + min(r, rows - 1);
            Ls[r] = r < rows ? b.lse[jq * b.P + pair] : INFINITY;
            Ds[r] = b.delta[jq * b.P + pair];
        }
        lds_fence_barrier_bwd();
        if (!active) continue;
        for (int c32 = 0; c32 < rows; c32 += 32) {
            f32x16 sc, dp;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                sc[e] = 0.f;
                dp[e] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&Qs[(c32 + arow) * STR + 16 * i + 8 * g]);
                const bf16x8 aa = *reinterpret_cast<const bf16x8*>(&As[(c32 + arow) * STR + 16 * i + 8 * g]);
                const bf16x8 al = *reinterpret_cast<const bf16x8*>(&Al[(c32 + arow) * STR + 16 * i + 8 * g]);
                sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kop[i], sc, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, vop[i], dp, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aa, vop[i], dp, 0, 0, 0);
            }
            // element e holds query c32 + (e&7) + 8g + 16(e>>3)
            const float4 l0 = *reinterpret_cast<const float4*>(&Ls[c32 + 8 * g]);
            const float4 l1 = *reinterpret_cast<const float4*>(&Ls[c32 + 8 * g + 4]);
            const float4 l2 = *reinterpret_cast<const float4*>(&Ls[c32 + 16 + 8 * g]);
            const float4 l3 = *reinterpret_cast<const float4*>(&Ls[c32 + 16 + 8 * g + 4]);
            const float4 e0 = *reinterpret_cast<const float4*>(&Ds[c32 + 8 * g]);
            const float4 e1 = *reinterpret_cast<const float4*>(&Ds[c32 + 8 * g + 4]);
            const float4 e2 = *reinterpret_cast<const float4*>(&Ds[c32 + 16 + 8 * g]);
            const float4 e3 = *reinterpret_cast<const float4*>(&Ds[c32 + 16 + 8 * g + 4]);
            const float lv[16] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w,
                                  l2.x, l2.y, l2.z, l2.w, l3.x, l3.y, l3.z, l3.w};
            const float dv[16] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w,
                                  e2.x, e2.y, e2.z, e2.w, e3.x, e3.y, e3.z, e3.w};
            // dS as two bf16 terms each (the rounded value and its rounding error), as
            // in the query side
            bf16x8 p0, p1, s0, s1, r0, r1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pa = fast_exp2(__builtin_fmaf(sc[e], sigma2, -lv[e]));
                const float pb = fast_exp2(__builtin_fmaf(sc[e + 8], sigma2, -lv[e + 8]));
                p0[e] = (bf16)pa;
                p1[e] = (bf16)pb;
                const float da = pa * (dp[e] - dv[e]), db = pb * (dp[e + 8] - dv[e + 8]);
                s0[e] = (bf16)da;
                s1[e] = (bf16)db;
                r0[e] = (bf16)(da - (float)s0[e]);
                r1[e] = (bf16)(db - (float)s1[e]);
            }
            const bf16* a_lo = &At[kl * STR + c32 + 8 * g];
            const bf16* a_hi = &At[(32 + kl) * STR + c32 + 8 * g];
            const bf16* q_lo = &Qt[kl * STR + c32 + 8 * g];
            const bf16* q_hi = &Qt[(32 + kl) * STR + c32 + 8 * g];
            dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a_lo), p0, dv0, 0, 0, 0);
            dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a_lo + 16), p1, dv0, 0, 0, 0);
            dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a_hi), p0, dv1, 0, 0, 0);
            dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a_hi + 16), p1, dv1, 0, 0, 0);
            dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_lo), r0, dk0, 0, 0, 0);
            dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_lo + 16), r1, dk0, 0, 0, 0);
            dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_hi), r0, dk1, 0, 0, 0);
            dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_hi + 16), r1, dk1, 0, 0, 0);
            dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_lo), s0, dk0, 0, 0, 0);
            dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_lo + 16), s1, dk0, 0, 0, 0);
            dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_hi), s0, dk1, 0, 0, 0);
            dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(q_hi + 16), s1, dk1, 0, 0, 0);
        }
    }
    if (!kvalid) return;
    // the block's last row: this step's first visit when steps run in forward order
    const bool first = !b.kv_accumulate && krow_local == nkv - 1;
    float* kr = b.k_bar + i_row * slab + pair * DH;
    float* vr = b.v_bar + i_row * slab + pair * DH;
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int dh0 = blk * 32 + 8 * ee + 4 * g;
            const f32x16& kk = blk ? dk1 : dk0;
            const f32x16& vv = blk ? dv1 : dv0;
            float4 kx = make_float4(b.sigma * kk[4 * ee + 0], b.sigma * kk[4 * ee + 1], b.sigma * kk[4 * ee + 2],
                                    b.sigma * kk[4 * ee + 3]);
            float4 vx = make_float4(vv[4 * ee + 0], vv[4 * ee + 1], vv[4 * ee + 2], vv[4 * ee + 3]);
            float4* kp = reinterpret_cast<float4*>(kr + dh0);
            float4* vp = reinterpret_cast<float4*>(vr + dh0);
            if (!first) {
                const float4 ko = *kp, vo = *vp;
                kx.x += ko.x; kx.y += ko.y; kx.z += ko.z; kx.w += ko.w;
                vx.x += vo.x; vx.y += vo.y; vx.z += vo.z; vx.w += vo.w;
            }
            *kp = kx;
            *vp = vx;
        }
    }
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
    hipLaunchKernelGGL((bwd_step_kernel<T, DH>), grid_for((int64_t)(nkv + nq) * b.P, DH), dim3(256), 0, s, b, kv0,
                       nkv, q0, nq);
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

template <int WAVES>
static hipError_t step_mfma(const BackwardArgs& b, int32_t kv0, int32_t nkv, int32_t q0, int32_t nq, hipStream_t s) {
    const int nkt = (nkv + 32 * WAVES - 1) / (32 * WAVES), nqt = (nq + 32 * WAVES - 1) / (32 * WAVES);
    hipLaunchKernelGGL((bwd_kv_mfma_kernel<WAVES>), dim3((uint32_t)(b.P * nkt)), dim3(64 * WAVES), 0, s, b, kv0, nkv,
                       q0, nq, nkt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_q_mfma_kernel<WAVES>), dim3((uint32_t)(b.P * nqt)), dim3(64 * WAVES), 0, s, b, kv0, nkv,
                       q0, nq, nqt);
    return hipGetLastError();
}

hipError_t launch_backward_step(rt_dtype dt, int head_dim, const BackwardArgs& b, int32_t kv0, int32_t nkv,
                                int32_t q0, int32_t nq, hipStream_t s) {
    if (nkv <= 0 || nq <= 0) return hipSuccess;
    // blocks of 32 pairs and more (powers of two in the blocked schedule): MFMA rectangles
    // (blocks of 16 measured no faster there than on the SIMT kernel)
    if (dt == RT_BF16 && head_dim == 64 && nkv >= 32 && nkv % 32 == 0) {
        const int w = nkv >= 128 ? 4 : (nkv >= 64 ? 2 : 1);  // waves per workgroup on the key side
        return w == 4 ? step_mfma<4>(b, kv0, nkv, q0, nq, s)
                      : (w == 2 ? step_mfma<2>(b, kv0, nkv, q0, nq, s) : step_mfma<1>(b, kv0, nkv, q0, nq, s));
    }
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
