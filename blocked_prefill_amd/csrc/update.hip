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

// Step s of a launch that runs several steps of one level (UpdateArgs::n_steps).
// The steps of one level touch distinct query rows: step t's rows t+1..t+b lie
// between consecutive odd multiples of b.
__device__ __forceinline__ UpdateArgs level_step(const UpdateArgs& in, int s) {
    UpdateArgs a = in;
    if (s > 0) {
        const int32_t shift = s * 2 * in.nkv;
        a.kv0 += shift;
        a.q0 += shift;
        a.nq = min(in.nkv, in.n_pos - a.q0);
        a.init = 0;
        a.a_out = (char*)in.a_out + (int64_t)s * in.a_step;
    }
    return a;
}

// SIMT update: one item = (query row i, batch*head pair p), handled by a
// group of DH/8 consecutive lanes, each holding 8 of the DH components.
// Items are ordered pair-fastest, so neighbouring groups read neighbouring
// 16-byte pieces of the position-major q / k / v / state slabs.
// CAUSAL: plain causal attention, as in the MFMA kernel below.
template <typename T, int DH, bool CAUSAL>
__global__ __launch_bounds__(256) void update_simt_kernel(UpdateArgs a_in) {
    const UpdateArgs a = level_step(a_in, blockIdx.y);
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
    const int nkv = CAUSAL ? (int)j + 1 : a.nkv;
    for (int s = 0; s < nkv; ++s) {
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

    if constexpr (CAUSAL) {
        const float inv = 1.0f / lb;
#pragma unroll
        for (int e = 0; e < 8; ++e) ob[e] *= inv;
        store8((T*)a.a_out + j * slab + off, ob);
        return;
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
        if (a.lse && lane == 0) a.lse[j * a.P + p] = mn + log2f(lb);  // saved for the backward
    } else {
        if (lane == 0) {
            a.m[sidx] = mb;
            a.l[sidx] = lb;
        }
        store8(a.o + sidx * DH + lane * 8, ob);
    }
}

// SIMT update for the blocked schedule's smallest steps (blocks of U = 1, 2
// or 4 pairs), where a launch's time is the latency of its memory round
// trips. Items as in update_simt_kernel, with blockIdx.y the query row.
// One round trip per step: the code between the first load and the last
// merge has no branch, so the query, the U keys/values, the stored state and
// the ephemeral pair are all requested at once. Merges that do not apply (no
// stored state, no ephemeral pair) are merges of weight zero: their score is
// -inf, taken after the block's first key has made the running maximum
// finite, and their values are zeroed (their addresses fall back to the
// query's own, a valid location).
template <typename T, int DH, int U>
__device__ __forceinline__ void small_step(const UpdateArgs& a) {
    constexpr int G = DH / 8;
    const int64_t pg = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // pair * G + lane
    if (pg >= a.P * G) return;  // whole groups leave together
    const int64_t p = pg / G;
    const int lane = (int)(pg % G);
    const int64_t slab = a.P * DH;  // elements per position
    const int64_t off = p * DH + lane * 8;
    const T* kp = (const T*)a.k + (int64_t)a.kv0 * slab + off;
    const T* vp = (const T*)a.v + (int64_t)a.kv0 * slab + off;

    for (int64_t i = blockIdx.y; i < a.nq; i += gridDim.y) {
        const int64_t j = a.q0 + i;
        const int64_t sidx = j * a.P + p;
        const bool merge_state = !a.init;
        const bool finish = a.fin && i == 0;
        const T* qp = (const T*)a.q + j * slab + off;

        Raw8<T> qr, ker, ver, kr[U], vr[U];
        Raw8<float> osr;
        qr.load(qp);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            kr[u].load(kp + u * slab);
            vr[u].load(vp + u * slab);
        }
        const float* sp = merge_state ? a.m + sidx : (const float*)qp;
        const float* lp = merge_state ? a.l + sidx : (const float*)qp;
        const float ms_ld = *sp, ls_ld = *lp;
        osr.load(merge_state ? a.o + sidx * DH + lane * 8 : (const float*)a.q);
        ker.load(finish ? (const T*)a.k_eph + j * slab + off : qp);
        ver.load(finish ? (const T*)a.v_eph + j * slab + off : qp);

        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = qr[e] * a.sigma2;

        float mb = -INFINITY, lb = 0.f, ob[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        auto merge = [&](float d, const Raw8<T>& val) {
            const float mn = fmaxf(mb, d);
            const float c = fast_exp2(mb - mn);
            const float pe = fast_exp2(d - mn);
            lb = lb * c + pe;
#pragma unroll
            for (int e = 0; e < 8; ++e) ob[e] = ob[e] * c + pe * val[e];
            mb = mn;
        };
        auto score = [&](const Raw8<T>& key) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qv[e] * key[e];
            return group_sum<G>(d);
        };
#pragma unroll
        for (int u = 0; u < U; ++u) merge(score(kr[u]), vr[u]);  // the block (mb finite after u = 0)
        {  // the position's own ephemeral pair (weight zero unless finishing)
            const float d = score(ker);
            merge(finish ? d : -INFINITY, ver);
        }
        {  // the stored state (weight zero on first touch)
            const float ms = merge_state ? ms_ld : -INFINITY;
            const float ls = merge_state ? ls_ld : 0.f;
            const float mn = fmaxf(ms, mb);
            const float cs = fast_exp2(ms - mn), cb = fast_exp2(mb - mn);
            lb = ls * cs + lb * cb;
#pragma unroll
            for (int e = 0; e < 8; ++e) ob[e] = (merge_state ? osr[e] : 0.f) * cs + ob[e] * cb;
            mb = mn;
        }
        if (finish) {  // a = o / l
            const float inv = 1.0f / lb;
#pragma unroll
            for (int e = 0; e < 8; ++e) ob[e] *= inv;
            store8((T*)a.a_out + off, ob);
            if (a.lse && lane == 0) a.lse[sidx] = mb + log2f(lb);  // saved for the backward
        } else {
            if (lane == 0) {
                a.m[sidx] = mb;
                a.l[sidx] = lb;
            }
            store8(a.o + sidx * DH + lane * 8, ob);
        }
    }
}

template <typename T, int DH, int U>
__global__ __launch_bounds__(256) void update_small_kernel(UpdateArgs a) {
    small_step<T, DH, U>(level_step(a, blockIdx.z));
}

// The small steps of several sequences' layers in one launch (blockIdx.z picks
// the step; every step has the same block length U and pair count P, query
// counts may differ).
struct UpdateGroup {
    UpdateArgs a[kMaxUpdateGroup];
};

template <typename T, int DH, int U>
__global__ __launch_bounds__(256) void update_small_group_kernel(UpdateGroup g) {
    small_step<T, DH, U>(g.a[blockIdx.z]);
}

// Workgroup barrier ordering LDS accesses only: global loads stay in flight across it.
__device__ __forceinline__ void lds_fence_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// MFMA update for blocks of b >= 32 pairs (any length >= 32 with the RAGGED
// instance), head_dim 64, bf16 (gfx950).
//
// A workgroup of WAVES waves takes one (batch*head pair p, tile of 32*WAVES
// queries); each wave owns 32 queries. The block's keys and values stream
// through LDS in tiles of KT positions, shared by the waves:
//   S^T[kv][q] = K Q^T       v_mfma_f32_32x32x16_bf16, A = K rows, B = Q^T
//   O^T[dh][q] += V^T P^T    A = V^T (transposed into LDS), B = P^T
// With K's rows fed in an order that swaps bits 2 and 3 of the row index,
// the scores a lane holds for its query (lane % 32) cover 8 consecutive key
// positions per 16-position slice, which is exactly the B-operand layout of
// the second product: P never leaves registers, and the softmax statistics
// and the O^T rescale are lane-local (the two lanes q and q+32 share a query).
// Workgroups are dispatched so that each XCD takes one contiguous range of
// (pair, query tile) items: an XCD's concurrent workgroups read neighbouring
// 128-byte pieces of the position-major slabs, and all query tiles of a pair
// run on the same XCD back to back, keeping its keys/values in that L2.
// KT: key/value positions per LDS tile (32 or 64). V^T sits in LDS with its
// 8-key chunks XOR-swizzled by the dh row's 8-row group, so that the
// transposing stores of a wave fall into different banks.
//
// RAGGED: the block length need not be a multiple of 32 (decode, naive
// schedule); the missing key rows of the last chunk are masked.
// CAUSAL: plain causal attention (the Transformer layer's). Keys are the
// queries' own positions (kv0 = q0 = 0); query i takes key rows 0..i and is
// written to row i of a_out; no state is read or written.
template <int WAVES, int KT, bool RAGGED, bool CAUSAL>
// (four waves: at most 128 VGPRs, so that four waves share a SIMD)
__global__ __launch_bounds__(64 * WAVES, (WAVES == 4 ? 4 : 1)) void update_mfma_kernel(UpdateArgs a_in, int nqt) {
    const UpdateArgs a = level_step(a_in, blockIdx.y);
    if (a.nq <= 0) return;  // the whole workgroup
    constexpr int DH = 64;
    constexpr int KSTR = DH + 8;    // bf16 per K row in LDS (16-byte pad)
    constexpr int VSTR = KT + 8;    // bf16 per V^T row in LDS
    constexpr int NT = 64 * WAVES;
    // K and V^T tiles; after the key loop the same bytes hold each wave's
    // 32 x 32 fp32 transpose tile of the state rows (pitch TP floats)
    constexpr int TP = 36;
    constexpr int LDS_KV = (KT * KSTR + DH * VSTR) * 2, LDS_T = WAVES * 32 * TP * 4;
    __shared__ __attribute__((aligned(16))) char lds_raw[LDS_KV > LDS_T ? LDS_KV : LDS_T];
    bf16* const Ks = reinterpret_cast<bf16*>(lds_raw);
    bf16* const Vt = Ks + KT * KSTR;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, ql = lane & 31;

    int64_t pair;
    int qtile;
    {
        // workgroup i runs on XCD i % 8; the grid (P * nqt items) divides by 8 when P does
        const int64_t i = blockIdx.x;
        const int64_t item = (a.P & 7) == 0 ? (i & 7) * ((int64_t)gridDim.x >> 3) + (i >> 3) : i;
        pair = item / nqt;
        qtile = (int)(item % nqt);
    }
    const int64_t slab = a.P * DH;
    const int wave_q0 = qtile * 32 * WAVES + wave * 32;
    const bool wave_active = wave_q0 < a.nq;
    const int qrow = wave_q0 + ql;
    // keys of this block: a causal tile needs those up to its last query
    const int nkv = CAUSAL ? min(a.nq, (qtile + 1) * 32 * WAVES) : a.nkv;
    const bool qvalid = qrow < a.nq;
    const int64_t j = (int64_t)a.q0 + qrow;

    bf16x8 qop[4];
    if (qvalid) {
        const bf16* qp = (const bf16*)a.q + j * slab + pair * DH + 8 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) qop[i] = *reinterpret_cast<const bf16x8*>(qp + 16 * i);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) qop[i][e] = (bf16)0.f;
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x16 o0, o1;  // O^T, dh 0..31 and 32..63
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        o0[e] = 0.f;
        o1[e] = 0.f;
    }
    const bf16* kbase = (const bf16*)a.k + (int64_t)a.kv0 * slab + pair * DH;
    const bf16* vbase = (const bf16*)a.v + (int64_t)a.kv0 * slab + pair * DH;
    // this lane's K row within a 32-row chunk: bits 2 and 3 swapped
    const int krow = (ql & ~12) | ((ql & 4) << 1) | ((ql & 8) >> 1);
    const float sigma2 = a.sigma2;

    // K/V tiles are fetched into registers one tile ahead: tile i+1's loads are
    // in flight while tile i is multiplied (LDS-only barriers keep them in flight).
    constexpr int KCH = KT * 8 / NT;        // 16-byte K chunks per thread per tile
    constexpr int VCH = (KT / 2) * 8 / NT;  // V row-pair chunks per thread per tile
    static_assert(KCH >= 1 && VCH >= 1 && (KT * 8) % NT == 0 && ((KT / 2) * 8) % NT == 0, "tile staging");
    static_assert(KT == 32 || KT == 64, "key tile");
    // whole tiles (the plain instance: the host guarantees nkv % KT == 0) are
    // read at per-thread 32-bit byte offsets from the tile's first row
    const uint32_t row_bytes = (uint32_t)(slab * 2);
    uint32_t koff[KCH], voff[VCH];
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
        const int c = tid + NT * i;
        koff[i] = (uint32_t)(c >> 3) * row_bytes + (uint32_t)(c & 7) * 16;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
        const int c = tid + NT * i;
        voff[i] = (uint32_t)((c >> 3) * 2) * row_bytes + (uint32_t)(c & 7) * 16;
    }
    bf16x8 kreg[KCH], vreg[VCH][2];
    auto fetch = [&](int kt0) {
        if constexpr (RAGGED || CAUSAL) {
            // rows past the block (a ragged last tile) repeat its last row: real,
            // finite data whose scores are masked (weight exactly 0). The loads are
            // unconditional so that they stay in flight across the tile's work.
            const int last = ((nkv - kt0) < KT ? (nkv - kt0) : KT) - 1;
#pragma unroll
            for (int i = 0; i < KCH; ++i) {
                const int c = tid + NT * i, r = min(c >> 3, last), ch = (c & 7) * 8;
                kreg[i] = *reinterpret_cast<const bf16x8*>(kbase + (int64_t)(kt0 + r) * slab + ch);
            }
#pragma unroll
            for (int i = 0; i < VCH; ++i) {
                const int c = tid + NT * i, r0 = (c >> 3) * 2, ch = (c & 7) * 8;
                vreg[i][0] = *reinterpret_cast<const bf16x8*>(vbase + (int64_t)(kt0 + min(r0, last)) * slab + ch);
                vreg[i][1] = *reinterpret_cast<const bf16x8*>(vbase + (int64_t)(kt0 + min(r0 + 1, last)) * slab + ch);
            }
        } else {
            const char* kb = (const char*)(kbase + (int64_t)kt0 * slab);
            const char* vb = (const char*)(vbase + (int64_t)kt0 * slab);
#pragma unroll
            for (int i = 0; i < KCH; ++i) kreg[i] = *reinterpret_cast<const bf16x8*>(kb + koff[i]);
#pragma unroll
            for (int i = 0; i < VCH; ++i) {
                vreg[i][0] = *reinterpret_cast<const bf16x8*>(vb + voff[i]);
                vreg[i][1] = *reinterpret_cast<const bf16x8*>(vb + voff[i] + row_bytes);
            }
        }
    };
    // V^T element (dh row d, key column kc): the 8-key chunk index is XORed with (d / 8) % (KT / 8)
    auto vt_at = [](int d, int kc) { return d * VSTR + ((((kc >> 3) ^ ((d >> 3) & (KT / 8 - 1)))) << 3) + (kc & 7); };
    fetch(0);
    for (int kt0 = 0; kt0 < nkv; kt0 += KT) {
        const int rows = (nkv - kt0) < KT ? (nkv - kt0) : KT;  // 1..64 (64 except the last tile)
        lds_fence_barrier();  // the previous tile's LDS reads are done
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int c = tid + NT * i, r = c >> 3, ch = (c & 7) * 8;
            *reinterpret_cast<bf16x8*>(&Ks[r * KSTR + ch]) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int c = tid + NT * i, r0 = (c >> 3) * 2, ch = (c & 7) * 8;
            {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
                    bf16x2 w;
                    w[0] = vreg[i][0][e];
                    w[1] = vreg[i][1][e];
                    *reinterpret_cast<bf16x2*>(&Vt[vt_at(ch + e, r0)]) = w;
                }
            }
        }
        lds_fence_barrier();  // this tile is in LDS
        if (kt0 + KT < nkv) fetch(kt0 + KT);
        if (!wave_active) continue;
        for (int c32 = 0; c32 < rows; c32 += 32) {
            if (CAUSAL && kt0 + c32 > wave_q0 + 31) break;  // past this wave's last query
            f32x16 s;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&Ks[(c32 + krow) * KSTR + 16 * i + 8 * g]);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[i], s, 0, 0, 0);
            }
            // running maximum on the raw scores (softmax_scale >= 0, so the
            // scaled maximum is sigma2 times it); the reference point m_run only
            // moves when some query's maximum exceeds it by more than 8 (base 2),
            // so the O^T rescale is skipped by the whole wave most of the time.
            // Masking (RAGGED: key rows at or past the block's end; CAUSAL: also
            // keys after the lane's query) exists only in those instances: the
            // blocked schedule's blocks are whole 32-row chunks.
            uint32_t live = 0xffffu;  // bit e: score e is a real key
            if constexpr (RAGGED || CAUSAL) {
                const bool masked = CAUSAL ? kt0 + c32 + 31 > wave_q0 : c32 + 32 > rows;  // wave-uniform
                if (masked) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int kv = c32 + (e & 7) + 8 * g + 16 * (e >> 3);  // key row of score e (see krow)
                        const bool dead = CAUSAL ? (kt0 + kv > qrow || kt0 + kv >= nkv) : kv >= rows;
                        if (dead) {
                            s[e] = -INFINITY;
                            live &= ~(1u << e);
                        }
                    }
                }
            }
            // this lane's half of the query's scores first: the two halves are
            // combined (a cross-lane exchange) only when some lane's half would
            // move the reference point; max(a, b)*sigma2 = max(a*sigma2, b*sigma2)
            // exactly for sigma2 >= 0, so the decisions equal those on the whole row
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[e]);
            mx *= sigma2;
            if (__builtin_amdgcn_ballot_w64(!(mx <= m_run + 8.0f))) {  // also true while m_run is -inf
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                const bool move = !(mx <= m_run + 8.0f);
                const float m_new = move ? fmaxf(m_run, mx) : m_run;
                const float alpha = fast_exp2(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    o0[e] *= alpha;
                    o1[e] *= alpha;
                }
                m_run = m_new;
            }
            float ps = 0.f;
            bf16x8 p0, p1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float pa = fast_exp2(__builtin_fmaf(s[e], sigma2, -m_run));
                float pb = fast_exp2(__builtin_fmaf(s[e + 8], sigma2, -m_run));
                if constexpr (RAGGED || CAUSAL) {  // (zero also when softmax_scale is 0)
                    if (!(live & (1u << e))) pa = 0.f;
                    if (!(live & (1u << (e + 8)))) pb = 0.f;
                }
                ps += pa + pb;
                p0[e] = (bf16)pa;
                p1[e] = (bf16)pb;
            }
            l_run += ps;  // this lane's half of the row sum; the halves are added after the loop
            const bf16x8 vlo0 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(ql, c32 + 8 * g)]);
            const bf16x8 vlo1 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(ql, c32 + 8 * g + 16)]);
            const bf16x8 vhi0 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(32 + ql, c32 + 8 * g)]);
            const bf16x8 vhi1 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(32 + ql, c32 + 8 * g + 16)]);
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vlo0, p0, o0, 0, 0, 0);
            o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vlo1, p1, o0, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhi0, p0, o1, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhi1, p1, o1, 0, 0, 0);
        }
    }
    l_run += __shfl_xor(l_run, 32, 64);  // the two halves of each query's row sum

    // this lane holds dh = blk*32 + 8*ee + 4*g + (0..3) for blk in {0,1}, ee in 0..3 (accumulator e = 4*ee + i)
    if constexpr (CAUSAL) {
        if (!qvalid) return;
        const float inv = 1.0f / l_run;
        bf16* out = (bf16*)a.a_out + j * slab + pair * DH;
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int dh0 = blk * 32 + 8 * ee + 4 * g;
                bf16x4 r;
#pragma unroll
                for (int i = 0; i < 4; ++i) r[i] = (bf16)((blk ? o1[4 * ee + i] : o0[4 * ee + i]) * inv);
                *reinterpret_cast<bf16x4*>(out + dh0) = r;
            }
        }
        return;
    }
    // Merge with the stored state: new = stored * cs + this block's * cb.
    const int64_t sidx = j * a.P + pair;
    const bool fin_row = a.fin && qrow == 0;
    float cs = 0.f, cb = 1.f;
    if (!a.init && qvalid) {
        const float ms = a.m[sidx], ls = a.l[sidx];
        const float m_new = fmaxf(ms, m_run);
        cs = fast_exp2(ms - m_new);
        cb = fast_exp2(m_run - m_new);
        l_run = ls * cs + l_run * cb;
        m_run = m_new;
    }
    // the stored numerator of the finishing row (the only row merged in registers)
    auto merge_regs = [&]() {
        const float* orow = a.o + sidx * DH;
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
            const float4 s0 = *reinterpret_cast<const float4*>(orow + 8 * ee + 4 * g);
            const float4 s1 = *reinterpret_cast<const float4*>(orow + 32 + 8 * ee + 4 * g);
            o0[4 * ee + 0] = s0.x * cs + o0[4 * ee + 0] * cb;
            o0[4 * ee + 1] = s0.y * cs + o0[4 * ee + 1] * cb;
            o0[4 * ee + 2] = s0.z * cs + o0[4 * ee + 2] * cb;
            o0[4 * ee + 3] = s0.w * cs + o0[4 * ee + 3] * cb;
            o1[4 * ee + 0] = s1.x * cs + o1[4 * ee + 0] * cb;
            o1[4 * ee + 1] = s1.y * cs + o1[4 * ee + 1] * cb;
            o1[4 * ee + 2] = s1.z * cs + o1[4 * ee + 2] * cb;
            o1[4 * ee + 3] = s1.w * cs + o1[4 * ee + 3] * cb;
        }
    };
    if (qvalid && !fin_row && g == 0) {
        a.m[sidx] = m_run;
        a.l[sidx] = l_run;
    }
    {
        // The fp32 numerator rows (256 bytes per query, about half of a step's
        // bytes) go through LDS so that they are read and written as whole
        // 128-byte lines. Each wave writes its O^T, 32 dh at a time, transposed
        // into its tile; then each 8 lanes move one query's 32 values (b = 64
        // 128.7 -> 116.3 us per step, b = 128 247 -> 221, b = 256 491 -> 453,
        // against each lane's 16-byte pieces of 32 rows).
        lds_fence_barrier();  // every wave is done with the K/V tiles
        float* tw = reinterpret_cast<float*>(lds_raw) + wave * 32 * TP;
        if (g == 0) tw[ql * TP + 32] = cs;  // each query's cs, in the tile's padding column
        const int rr = lane >> 3, cc = (lane & 7) * 4;  // this lane's row (of 8 per pass) and 4 columns
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            // lane (ql, g) holds dh = blk*32 + 8*ee + 4*g + i of query ql
#pragma unroll
            for (int ee = 0; ee < 4; ++ee)
                *reinterpret_cast<float4*>(&tw[ql * TP + 8 * ee + 4 * g]) =
                    blk ? make_float4(o1[4 * ee] * cb, o1[4 * ee + 1] * cb, o1[4 * ee + 2] * cb, o1[4 * ee + 3] * cb)
                        : make_float4(o0[4 * ee] * cb, o0[4 * ee + 1] * cb, o0[4 * ee + 2] * cb, o0[4 * ee + 3] * cb);
#pragma unroll
            for (int pass = 0; pass < 4; ++pass) {
                const int r = pass * 8 + rr, row = wave_q0 + r;
                float4 v = *reinterpret_cast<const float4*>(&tw[r * TP + cc]);
                if (row < a.nq && !(a.fin && row == 0)) {
                    float* op = a.o + ((int64_t)(a.q0 + row) * a.P + pair) * DH + blk * 32 + cc;
                    if (!a.init) {
                        const float c = tw[r * TP + 32];
                        const float4 sv = *reinterpret_cast<const float4*>(op);
                        v = make_float4(sv.x * c + v.x, sv.y * c + v.y, sv.z * c + v.z, sv.w * c + v.w);
                    }
                    *reinterpret_cast<float4*>(op) = v;
                }
            }
        }
        if (!fin_row || !qvalid) return;
        if (!a.init) merge_regs();
    }
    {
        // the position's own ephemeral pair (lanes 0 and 32 hold the two halves of the query)
        const bf16* kp = (const bf16*)a.k_eph + j * slab + pair * DH + 8 * g;
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kp + 16 * i);
#pragma unroll
            for (int e = 0; e < 8; ++e) d += (float)qop[i][e] * (float)kv[e];
        }
        d += __shfl_xor(d, 32, 64);
        d *= sigma2;
        const float m_new = fmaxf(m_run, d);
        const float c = fast_exp2(m_run - m_new), pe = fast_exp2(d - m_new);
        const float inv = 1.0f / (l_run * c + pe);
        if (a.lse && g == 0) a.lse[j * a.P + pair] = m_new + log2f(l_run * c + pe);  // saved for the backward
        const bf16* vp = (const bf16*)a.v_eph + j * slab + pair * DH;
        bf16* out = (bf16*)a.a_out + pair * DH;
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int dh0 = blk * 32 + 8 * ee + 4 * g;
                const bf16x4 ve = *reinterpret_cast<const bf16x4*>(vp + dh0);
                bf16x4 r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ov = blk ? o1[4 * ee + i] : o0[4 * ee + i];
                    r[i] = (bf16)((ov * c + pe * (float)ve[i]) * inv);
                }
                *reinterpret_cast<bf16x4*>(out + dh0) = r;
            }
        }
    }
}

// MFMA update for blocks of 16 (PPW = 2) or 8 (PPW = 4) pairs (bf16, head_dim
// 64): one wave takes PPW = 32 / b neighbouring (batch*head) pairs at once. Its 32 key rows
// are the b keys of each of its pairs and its 32 query columns the (up to b)
// queries of each, so the two products of the large-block kernel, S^T = K Q^T
// and O^T = V^T P^T, apply unchanged; a score counts only where its key row
// and query column belong to the same pair (the other products get weight 0).
// A lane holds 16 scores of its query, of which the 8 of one 16-key slice can
// be its pair's: with PPW = 2 the slice is the pair's index, with PPW = 4 the
// pair's rows sit in one 8-row group of one slice, held by one of the query's
// two lanes. One key/value tile, no running maximum; the stored state is
// fetched together with the tile.
template <int PPW>
__global__ __launch_bounds__(64) void update_mfma_multi_kernel(UpdateArgs a_in) {
    const UpdateArgs a = level_step(a_in, blockIdx.y);
    constexpr int DH = 64, KB = 32 / PPW;  // keys (and at most as many queries) per pair
    constexpr int KSTR = DH + 8, VSTR = 32 + 8;
    static_assert(PPW == 2 || PPW == 4, "pairs per wave");
    __shared__ __attribute__((aligned(16))) bf16 Ks[32 * KSTR];
    __shared__ __attribute__((aligned(16))) bf16 Vt[DH * VSTR];
    const int lane = threadIdx.x, g = lane >> 5, ql = lane & 31;
    const int64_t wi = blockIdx.x;
    // each XCD (workgroup i runs on XCD i % 8) takes a contiguous range of pair groups
    const int64_t item = (gridDim.x & 7) == 0 ? (wi & 7) * ((int64_t)gridDim.x >> 3) + (wi >> 3) : wi;
    const int64_t pair0 = item * PPW;
    const int pi = ql / KB, qi = ql % KB;
    const int64_t pair = pair0 + pi;
    const int64_t slab = a.P * DH;
    const bool qvalid = qi < a.nq;
    const int64_t j = (int64_t)a.q0 + (qvalid ? qi : 0);  // an invalid column reads row q0; its result is dropped
    const int64_t sidx = j * a.P + pair;

    // every load up front, unconditionally: keys/values, the query, the stored state
    const bf16* kb = (const bf16*)a.k + (int64_t)a.kv0 * slab + pair0 * DH;
    const bf16* vb = (const bf16*)a.v + (int64_t)a.kv0 * slab + pair0 * DH;
    bf16x8 kreg[4], vreg[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // K row r = (pair r / KB, key r % KB), 16-byte chunk c % 8
        const int c = lane + 64 * i, r = c >> 3, ch = (c & 7) * 8;
        kreg[i] = *reinterpret_cast<const bf16x8*>(kb + (int64_t)(r % KB) * slab + (r / KB) * DH + ch);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // V rows r0, r0 + 1 (one pair: KB is even)
        const int c = lane + 64 * i, r0 = (c >> 3) * 2, ch = (c & 7) * 8;
        vreg[i][0] = *reinterpret_cast<const bf16x8*>(vb + (int64_t)(r0 % KB) * slab + (r0 / KB) * DH + ch);
        vreg[i][1] = *reinterpret_cast<const bf16x8*>(vb + (int64_t)((r0 + 1) % KB) * slab + ((r0 + 1) / KB) * DH + ch);
    }
    bf16x8 qop[4];
    {
        const bf16* qp = (const bf16*)a.q + j * slab + pair * DH + 8 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) qop[i] = *reinterpret_cast<const bf16x8*>(qp + 16 * i);
    }
    // a first visit (init) has no stored state (m, l, o may be null, as in a
    // decode step): its loads then read the tile's first key row instead (the
    // PPW pairs' keys there span at least 256 bytes) and are not used
    const float* m_ld = a.init ? (const float*)kb : a.m + sidx;
    const float* l_ld = a.init ? (const float*)kb : a.l + sidx;
    const float* o_ld = a.init ? (const float*)kb : a.o + sidx * DH;
    const float ms = *m_ld, ls = *l_ld;
    float4 os[8];
#pragma unroll
    for (int ee = 0; ee < 4; ++ee) {
        os[ee] = *reinterpret_cast<const float4*>(o_ld + 8 * ee + 4 * g);
        os[4 + ee] = *reinterpret_cast<const float4*>(o_ld + 32 + 8 * ee + 4 * g);
    }

    // V^T chunk swizzle as in the large-block kernel (32-key tile)
    auto vt_at = [](int d, int kc) { return d * VSTR + ((((kc >> 3) ^ ((d >> 3) & 3))) << 3) + (kc & 7); };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = lane + 64 * i, r = c >> 3, ch = (c & 7) * 8;
        *reinterpret_cast<bf16x8*>(&Ks[r * KSTR + ch]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = lane + 64 * i, r0 = (c >> 3) * 2, ch = (c & 7) * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
            bf16x2 w;
            w[0] = vreg[i][0][e];
            w[1] = vreg[i][1][e];
            *reinterpret_cast<bf16x2*>(&Vt[vt_at(ch + e, r0)]) = w;
        }
    }
    lds_fence_barrier();

    const int krow = (ql & ~12) | ((ql & 4) << 1) | ((ql & 8) >> 1);  // bits 2 and 3 swapped
    f32x16 sc;
#pragma unroll
    for (int e = 0; e < 16; ++e) sc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(&Ks[krow * KSTR + 16 * i + 8 * g]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[i], sc, 0, 0, 0);
    }
    // score e of this lane is key row (e % 8) + 8 g + 16 (e / 8), i.e. pair g + 2 (e / 8) for
    // 8-key pairs and pair e / 8 for 16-key pairs
    const int slice = PPW == 2 ? pi : (pi >> 1);
    const bool lane_ok = PPW == 2 || g == (pi & 1);
    float sel[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = slice ? sc[e + 8] : sc[e];
    float mx = -INFINITY;
    if (lane_ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sel[e]);
    }
    const float sigma2 = a.sigma2;
    float m_run = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sigma2;  // softmax_scale >= 0
    float pv[8], ps = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pv[e] = lane_ok ? fast_exp2(__builtin_fmaf(sel[e], sigma2, -m_run)) : 0.f;
        ps += pv[e];
    }
    float l_run = ps + __shfl_xor(ps, 32, 64);
    // P enters the second product as two bf16 terms, p = hi + lo (hi the bf16
    // rounding of p, lo that of the remainder), so the weights keep ~16
    // significant bits as in the fp32 SIMT kernel; the product's pipe is
    // otherwise idle in this memory-bound kernel
    bf16x8 p0, p1, r0, r1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 hi = (bf16)pv[e];
        const bf16 lo = (bf16)(pv[e] - (float)hi);
        const bf16 z = (bf16)0.f;
        p0[e] = slice == 0 ? hi : z;
        p1[e] = slice == 1 ? hi : z;
        r0[e] = slice == 0 ? lo : z;
        r1[e] = slice == 1 ? lo : z;
    }
    f32x16 o0, o1;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        o0[e] = 0.f;
        o1[e] = 0.f;
    }
    {
        const bf16x8 vlo0 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(ql, 8 * g)]);
        const bf16x8 vlo1 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(ql, 8 * g + 16)]);
        const bf16x8 vhi0 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(32 + ql, 8 * g)]);
        const bf16x8 vhi1 = *reinterpret_cast<const bf16x8*>(&Vt[vt_at(32 + ql, 8 * g + 16)]);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vlo0, r0, o0, 0, 0, 0);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vlo1, r1, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhi0, r0, o1, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhi1, r1, o1, 0, 0, 0);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vlo0, p0, o0, 0, 0, 0);
        o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vlo1, p1, o0, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhi0, p0, o1, 0, 0, 0);
        o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vhi1, p1, o1, 0, 0, 0);
    }
    if (!qvalid) return;

    // this lane holds dh = blk*32 + 8*ee + 4*g + (0..3) (accumulator e = 4*ee + i), as in the large-block kernel
    if (!a.init) {
        const float m_new = fmaxf(ms, m_run);
        const float cs = fast_exp2(ms - m_new), cb = fast_exp2(m_run - m_new);
        l_run = ls * cs + l_run * cb;
        m_run = m_new;
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
            o0[4 * ee + 0] = os[ee].x * cs + o0[4 * ee + 0] * cb;
            o0[4 * ee + 1] = os[ee].y * cs + o0[4 * ee + 1] * cb;
            o0[4 * ee + 2] = os[ee].z * cs + o0[4 * ee + 2] * cb;
            o0[4 * ee + 3] = os[ee].w * cs + o0[4 * ee + 3] * cb;
            o1[4 * ee + 0] = os[4 + ee].x * cs + o1[4 * ee + 0] * cb;
            o1[4 * ee + 1] = os[4 + ee].y * cs + o1[4 * ee + 1] * cb;
            o1[4 * ee + 2] = os[4 + ee].z * cs + o1[4 * ee + 2] * cb;
            o1[4 * ee + 3] = os[4 + ee].w * cs + o1[4 * ee + 3] * cb;
        }
    }
    if (a.fin && qi == 0) {
        // the position's own ephemeral pair (lanes ql and ql + 32 hold the two halves of the query)
        const bf16* kp = (const bf16*)a.k_eph + j * slab + pair * DH + 8 * g;
        float d = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 kv = *reinterpret_cast<const bf16x8*>(kp + 16 * i);
#pragma unroll
            for (int e = 0; e < 8; ++e) d += (float)qop[i][e] * (float)kv[e];
        }
        d += __shfl_xor(d, 32, 64);
        d *= sigma2;
        const float m_new = fmaxf(m_run, d);
        const float c = fast_exp2(m_run - m_new), pe = fast_exp2(d - m_new);
        const float inv = 1.0f / (l_run * c + pe);
        if (a.lse && g == 0) a.lse[sidx] = m_new + log2f(l_run * c + pe);  // saved for the backward
        const bf16* vp = (const bf16*)a.v_eph + j * slab + pair * DH;
        bf16* out = (bf16*)a.a_out + pair * DH;
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int dh0 = blk * 32 + 8 * ee + 4 * g;
                const bf16x4 ve = *reinterpret_cast<const bf16x4*>(vp + dh0);
                bf16x4 r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ov = blk ? o1[4 * ee + i] : o0[4 * ee + i];
                    r[i] = (bf16)((ov * c + pe * (float)ve[i]) * inv);
                }
                *reinterpret_cast<bf16x4*>(out + dh0) = r;
            }
        }
    } else {
        float* orow = a.o + sidx * DH;
        if (g == 0) {
            a.m[sidx] = m_run;
            a.l[sidx] = l_run;
        }
#pragma unroll
        for (int ee = 0; ee < 4; ++ee) {
            *reinterpret_cast<float4*>(orow + 8 * ee + 4 * g) =
                make_float4(o0[4 * ee + 0], o0[4 * ee + 1], o0[4 * ee + 2], o0[4 * ee + 3]);
            *reinterpret_cast<float4*>(orow + 32 + 8 * ee + 4 * g) =
                make_float4(o1[4 * ee + 0], o1[4 * ee + 1], o1[4 * ee + 2], o1[4 * ee + 3]);
        }
    }
}

template <int WAVES, bool CAUSAL = false>
static hipError_t launch_mfma(const UpdateArgs& a, hipStream_t s) {
    const int nqt = (a.nq + 32 * WAVES - 1) / (32 * WAVES);
    const dim3 grid((uint32_t)(a.P * nqt), (uint32_t)(a.n_steps > 1 ? a.n_steps : 1)), block(64 * WAVES);
    // the plain instances address a tile's rows with 32-bit byte offsets
    const bool offsets_fit = (uint64_t)a.P * 64 * 2 * 64 <= 0xffffffffull;
    if constexpr (CAUSAL) {
        hipLaunchKernelGGL((update_mfma_kernel<WAVES, 64, false, true>), grid, block, 0, s, a, nqt);
    } else if (!offsets_fit) {
        hipLaunchKernelGGL((update_mfma_kernel<WAVES, 64, true, false>), grid, block, 0, s, a, nqt);
    } else if (a.nkv % 64 == 0) {
        hipLaunchKernelGGL((update_mfma_kernel<WAVES, 64, false, false>), grid, block, 0, s, a, nqt);
    } else if (WAVES <= 2 && a.nkv % 32 == 0) {
        // 32-row tiles (staged by at most 128 threads)
        if constexpr (WAVES <= 2) hipLaunchKernelGGL((update_mfma_kernel<WAVES, 32, false, false>), grid, block, 0, s, a, nqt);
    } else {
        hipLaunchKernelGGL((update_mfma_kernel<WAVES, 64, true, false>), grid, block, 0, s, a, nqt);
    }
    return hipGetLastError();
}

template <typename T, int DH, bool CAUSAL>
static hipError_t launch_simt(const UpdateArgs& a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    if constexpr (!CAUSAL && sizeof(T) == 2) {
        // blocks of 1, 2 and 4 pairs (most steps of the blocked schedule): one round trip
        if (a.nkv == 1 || a.nkv == 2 || a.nkv == 4) {
            const dim3 grid((uint32_t)((a.P * (DH / 8) + 255) / 256), (uint32_t)(a.nq < 65535 ? a.nq : 65535),
                            (uint32_t)(a.n_steps > 1 ? a.n_steps : 1));
            if (a.nkv == 1)
                hipLaunchKernelGGL((update_small_kernel<T, DH, 1>), grid, dim3(256), 0, s, a);
            else if (a.nkv == 2)
                hipLaunchKernelGGL((update_small_kernel<T, DH, 2>), grid, dim3(256), 0, s, a);
            else
                hipLaunchKernelGGL((update_small_kernel<T, DH, 4>), grid, dim3(256), 0, s, a);
            return hipGetLastError();
        }
    }
    const int64_t threads = (int64_t)a.nq * a.P * (DH / 8);
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((update_simt_kernel<T, DH, CAUSAL>), dim3((uint32_t)blocks, (uint32_t)(a.n_steps > 1 ? a.n_steps : 1)),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

template <typename T, bool CAUSAL>
static hipError_t launch_typed(int head_dim, const UpdateArgs& a, hipStream_t s) {
    switch (head_dim) {
        case 32: return launch_simt<T, 32, CAUSAL>(a, s);
        case 64: return launch_simt<T, 64, CAUSAL>(a, s);
        case 128: return launch_simt<T, 128, CAUSAL>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_update_small_group(rt_dtype dt, int head_dim, const UpdateArgs* us, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (n > kMaxUpdateGroup) {
        for (int i0 = 0; i0 < n; i0 += kMaxUpdateGroup) {
            const hipError_t e = launch_update_small_group(dt, head_dim, us + i0,
                                                           n - i0 < kMaxUpdateGroup ? n - i0 : kMaxUpdateGroup, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    const int U = us[0].nkv;
    if (dt != RT_BF16 || head_dim != 64 || !(U == 1 || U == 2 || U == 4)) return hipErrorInvalidValue;
    int64_t max_nq = 0;
    for (int i = 0; i < n; ++i) {
        if (us[i].nkv != U || us[i].P != us[0].P || us[i].nq < 0) return hipErrorInvalidValue;
        max_nq = us[i].nq > max_nq ? us[i].nq : max_nq;
    }
    if (max_nq == 0) return hipSuccess;
    UpdateGroup g{};
    for (int i = 0; i < n; ++i) g.a[i] = us[i];
    constexpr int DH = 64;
    const dim3 grid((uint32_t)((us[0].P * (DH / 8) + 255) / 256), (uint32_t)(max_nq < 65535 ? max_nq : 65535),
                    (uint32_t)n);
    if (U == 1)
        hipLaunchKernelGGL((update_small_group_kernel<bf16, DH, 1>), grid, dim3(256), 0, s, g);
    else if (U == 2)
        hipLaunchKernelGGL((update_small_group_kernel<bf16, DH, 2>), grid, dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((update_small_group_kernel<bf16, DH, 4>), grid, dim3(256), 0, s, g);
    return hipGetLastError();
}

// Blocks of at least this many pairs go to the MFMA kernel (bf16, head_dim 64).
constexpr int kMfmaMinBlock = 32;

hipError_t launch_update(rt_dtype dt, int head_dim, const UpdateArgs& a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    if (a.n_steps > 65535) return hipErrorInvalidConfiguration;  // grid y/z limit
    if (dt == RT_BF16 && head_dim == 64 && a.nkv == 16 && a.nq <= 16 && a.P % 2 == 0) {
        // blocks of 16: two pairs per MFMA wave (blocks of 8, four pairs per wave,
        // measured 14.2 us per step at 8192 pairs against the SIMT kernel's 13.6)
        hipLaunchKernelGGL((update_mfma_multi_kernel<2>), dim3((uint32_t)(a.P / 2), (uint32_t)(a.n_steps > 1 ? a.n_steps : 1)),
                           dim3(64), 0, s, a);
        return hipGetLastError();
    }
    if (dt == RT_BF16 && head_dim == 64 && a.nkv >= kMfmaMinBlock) {
        const int waves_needed = (a.nq + 31) / 32;
        if (waves_needed <= 1) return launch_mfma<1>(a, s);
        if (waves_needed <= 2) return launch_mfma<2>(a, s);
        return launch_mfma<4>(a, s);
    }
    return dt == RT_BF16 ? launch_typed<bf16, false>(head_dim, a, s) : launch_typed<float, false>(head_dim, a, s);
}

hipError_t launch_causal_attention(rt_dtype dt, int head_dim, const UpdateArgs& a, hipStream_t s) {
    if (a.nq <= 0) return hipSuccess;
    if (dt == RT_BF16 && head_dim == 64) return launch_mfma<4, true>(a, s);
    return dt == RT_BF16 ? launch_typed<bf16, true>(head_dim, a, s) : launch_typed<float, true>(head_dim, a, s);
}

}  // namespace rt
