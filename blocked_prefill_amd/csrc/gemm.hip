// Projection GEMMs of the RT layer: C = epilogue(A * W^T), W row-major [out][in].
//
// Reading note (lshu.cn/news/403416), translated paper section 2: every
// projection acts on an RMS-normalised vector. RMS(a) * W^T equals
// rstd(a) * (a * W^T) row by row, so the normalisation is fused: the
// product is scaled row by row in the epilogue, from sums of a^2 over whole
// rows (a product that normalises never splits K). Section 2.1: the MLP is
// W_2 GELU(W_1 .) and both branches are added to the residual stream, also
// fused here.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 / 16x16x32_bf16 on gfx950, fp32
// accumulation. K tiles reach a swizzled LDS tile either through registers
// (prefetched several tiles ahead, double-buffered LDS) or directly
// (global_load_lds into a ring of LDS stages). In bf16 layers the row sums of
// squares come as partial sums: of h and z from the producing GEMM's
// epilogue, of a layer input from a row pass (row_sumsq); a product given
// none sums its own A rows while it multiplies them. A weight gradient's
// reduction over rows runs as K ranges in one launch (launch_gemm_splitk),
// each writing a partial. fp32 path: plain SIMT, one thread per output (used
// by small fp32 layers).
#include <type_traits>

#include "rt_device.h"
#include "rt_internal.h"

namespace rt {

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erf(u) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-u^2),
// t = 1/(1 + p u), u >= 0, absolute error <= 1.5e-7; odd extension for u < 0.
__device__ __forceinline__ float erf_as(float u) {
    const float a = fabsf(u);
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * a);
    const float poly =
        t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float e = __builtin_amdgcn_exp2f(-a * a * 1.4426950408889634f);
    return copysignf(1.0f - poly * e, u);
}
// GELU with the Gaussian CDF: x/2 (1 + erf(x/sqrt 2)).
__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erf_as(x * 0.70710678118654752f)); }
// Its derivative: Phi(x) + x phi(x).
__device__ __forceinline__ float gelu_erf_grad(float x) {
    return 0.5f * (1.0f + erf_as(x * 0.70710678118654752f)) +
           x * __builtin_amdgcn_exp2f(-0.5f * x * x * 1.4426950408889634f) * 0.39894228040143268f;
}

template <int FLAGS, typename TR, typename TC>
__device__ __forceinline__ void epilogue_store(const GemmArgs& g, TC* C, int64_t row, int64_t col, float v,
                                               float rstd) {
    if (FLAGS & EPI_RMS) v *= rstd;
    if (FLAGS & EPI_GELU) v = gelu_erf(v);
    if (FLAGS & EPI_DGELU) v *= gelu_erf_grad(to_f32(((const TR*)g.R)[row * g.ldr + col]));
    if (FLAGS & EPI_RESID) v = to_f32(((const TR*)g.R)[row * g.ldr + col]) + g.rscale * v;
    C[row * g.ldc + (col % g.seg_n)] = from_f32<TC>(v);
}

// ---------------------------------------------------------------- bf16 MFMA, pipelined

// Workgroup barrier that orders LDS accesses only: global loads stay in
// flight across it (a full __syncthreads would wait for every outstanding load).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Slot of the 16-byte chunk c (0..7) of tile row r in LDS: rows of 128 bytes,
// chunks XOR-swizzled by (r/2)%8 so that 16 consecutive rows read at one
// chunk column fall in 16 different 4-bank groups.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Waits until at most n vector-memory loads of this wave are outstanding
// (loads complete in issue order), leaving the newer ones in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | 0x70 | 0xF00 | ((n >> 4) << 14));
}
// Barrier of the direct-to-LDS ring: this wave's LDS reads are complete and no
// memory access is moved across it by the compiler, while the global->LDS
// loads in flight into the other stages stay in flight (a release fence on
// LDS would wait for them too).
__device__ __forceinline__ void dma_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// A small blocked step (blocks of 1, 2 or 4 pairs) run by the workgroup that
// has just produced the newest key/value row of the block for `rows` batch
// rows of one head (kvs: row r holds k then v, 64 each, as stored). The same
// arithmetic, merge order and branch-free loads as the standalone small-step
// kernel of update.hip: block keys oldest first (the newest from kvs), then
// the position's ephemeral pair, then the stored state; one 8-lane group per
// (batch row, query row) item.
__device__ __forceinline__ void fused_small_step(const UpdateArgs& a, const bf16* kvs, int kvs_pitch, int64_t m0,
                                                 int rows, int64_t B, int head, int tid, int nthreads) {
    constexpr int DH = 64, G = 8;
    const int64_t H = a.P / B;
    const int64_t slab = a.P * DH;
    const int lane = tid & (G - 1);
    const int items = rows * a.nq;
    for (int it = tid / G; it < items; it += nthreads / G) {
        const int r = it % rows, i = it / rows;
        const int64_t p = (m0 + r) * H + head;
        const int64_t j = a.q0 + i;
        const int64_t sidx = j * a.P + p;
        const int64_t off = p * DH + lane * 8;
        const bool merge_state = !a.init;
        const bool finish = a.fin && i == 0;
        const bf16* qp = (const bf16*)a.q + j * slab + off;
        Raw8<bf16> qr, ker, ver, kn, vn;
        Raw8<float> osr;
        qr.load(qp);
        const float* sp = merge_state ? a.m + sidx : (const float*)qp;
        const float* lp = merge_state ? a.l + sidx : (const float*)qp;
        const float ms_ld = *sp, ls_ld = *lp;
        osr.load(merge_state ? a.o + sidx * DH + lane * 8 : (const float*)a.q);
        ker.load(finish ? (const bf16*)a.k_eph + j * slab + off : qp);
        ver.load(finish ? (const bf16*)a.v_eph + j * slab + off : qp);
        kn.load(kvs + r * kvs_pitch + lane * 8);
        vn.load(kvs + r * kvs_pitch + DH + lane * 8);
        float qv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = qr[e] * a.sigma2;
        float mb = -INFINITY, lb = 0.f, ob[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        auto merge = [&](float d, const Raw8<bf16>& val) {
            const float mn = fmaxf(mb, d);
            const float c = fast_exp2(mb - mn);
            const float pe = fast_exp2(d - mn);
            lb = lb * c + pe;
#pragma unroll
            for (int e = 0; e < 8; ++e) ob[e] = ob[e] * c + pe * val[e];
            mb = mn;
        };
        auto score = [&](const Raw8<bf16>& key) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d += qv[e] * key[e];
            return group_sum<G>(d);
        };
        for (int u = 0; u + 1 < a.nkv; ++u) {  // the block's older pairs, from the caches
            Raw8<bf16> ko, vo;
            ko.load((const bf16*)a.k + (int64_t)(a.kv0 + u) * slab + off);
            vo.load((const bf16*)a.v + (int64_t)(a.kv0 + u) * slab + off);
            merge(score(ko), vo);
        }
        merge(score(kn), vn);  // the newest pair, as just stored
        {
            const float d = score(ker);
            merge(finish ? d : -INFINITY, ver);
        }
        {
            const float msv = merge_state ? ms_ld : -INFINITY;
            const float lsv = merge_state ? ls_ld : 0.f;
            const float mn = fmaxf(msv, mb);
            const float cs = fast_exp2(msv - mn), cb = fast_exp2(mb - mn);
            lb = lsv * cs + lb * cb;
#pragma unroll
            for (int e = 0; e < 8; ++e) ob[e] = (merge_state ? osr[e] : 0.f) * cs + ob[e] * cb;
            mb = mn;
        }
        if (finish) {
            const float inv = 1.0f / lb;
#pragma unroll
            for (int e = 0; e < 8; ++e) ob[e] *= inv;
            store8((bf16*)a.a_out + off, ob);
            if (a.lse && lane == 0) a.lse[sidx] = mb + log2f(lb);
        } else {
            if (lane == 0) {
                a.m[sidx] = mb;
                a.l[sidx] = lb;
            }
            store8(a.o + sidx * DH + lane * 8, ob);
        }
    }
}

// C = epilogue(A * W^T) with A, W bf16 and K % 64 == 0, N % BN == 0.
// K tiles of 64 are fetched into registers D tiles ahead of use (a ring of
// D register stages, so D-1 tiles are in flight while one is multiplied),
// written to a double-buffered swizzled LDS tile, and multiplied with
// v_mfma_f32_32x32x16_bf16; each wave computes a (BM/WM) x (BN/WN) block.
// One LDS-only barrier per K tile.
//
// PIPE_DMA: the K tiles bypass the registers: each wave's 16-byte loads land
// in LDS directly (global_load_lds_dwordx4, the 64 lanes' data in 64
// consecutive slots, which are the same swizzled slots as above), in a ring of
// D stages: tile kt+D-1 is in flight while tile kt is multiplied, and no VGPRs
// are spent on staging, which leaves room for 256x256 tiles. Each stage is an array of its own: the compiler
// tracks LDS written by these loads per object, and with one array it would
// wait for every load in flight before each LDS read of the tile.
//
// KS > 1 splits K inside the workgroup: KS groups of WM*WN waves each run the
// pipeline above over their own contiguous K range, with their own LDS
// buffers, and the KS partial tiles are added in LDS before the epilogue. At
// the per-position shapes (M = batch) this multiplies the waves per tile and
// divides the serial K-loop length without any cross-workgroup reduction.
// k_off, c_off (elements): where A and W start along K and where C starts, beyond
// the argument set's own pointers (one K range of a split product).
template <typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN, int D, int MF, int KS>
__device__ __forceinline__ void gemm_pipe_body(const GemmArgs& g, const uint32_t bx, const uint32_t by,
                                               const int64_t k_off = 0, const int64_t c_off = 0) {
    // MF = 32: v_mfma_f32_32x32x16_bf16 blocks; MF = 16: v_mfma_f32_16x16x32_bf16 blocks
    // (four times as many independent accumulators for the same wave tile).
    static_assert(MF == 32 || MF == 16, "MFMA block");
    static_assert(KS == 1 || !(FLAGS & EPI_RMS), "the self-summed row norm needs the whole K range");
    constexpr int NTG = 64 * WM * WN;  // threads of one K group
    constexpr int NT = NTG * KS;
    constexpr int BK = 64;
    constexpr int TMW = BM / WM, TNW = BN / WN;
    constexpr int FM = TMW / MF, FN = TNW / MF;
    typedef typename std::conditional<MF == 32, f32x16, f32x4>::type acc_t;
    constexpr int AE = MF == 32 ? 16 : 4;  // accumulator elements per lane
    constexpr int A_CH = BM * (BK / 8), W_CH = BN * (BK / 8);  // 16-byte chunks per tile
    constexpr int LA = A_CH / NTG, LW = W_CH / NTG;             // chunks per thread per tile
    constexpr int STAGE = (A_CH + W_CH) * 16;
    static_assert(FM >= 1 && FN >= 1 && A_CH % NTG == 0 && W_CH % NTG == 0, "tile shape");
    static_assert(D >= 2, "prefetch depth");

    constexpr bool DMA = (FLAGS & PIPE_DMA) != 0;
    constexpr int NBUF = DMA ? D : 2;  // LDS stages per K group
    static_assert(!DMA || (KS == 1 && D >= 2 && (D - 2) * (LA + LW) < 64), "direct-to-LDS ring");
    __shared__ __attribute__((aligned(16))) char smem_all[DMA ? 16 : KS * NBUF * STAGE];
    // PIPE_DMA: each stage its own array, so that the compiler sees a stage's LDS reads and
    // another stage's global->LDS loads as distinct objects and waits for neither
    // the epilogue's fp32 tile passes use stage 0 alone: the largest pass of BM, BM/2 or BM/4
    // rows that fits in a quarter more than a stage sizes it
    constexpr int EPI_ROW = (BN + 4) * 4;
    constexpr int EPI_PR = BM * EPI_ROW <= STAGE * 5 / 4 ? BM : BM / 2 * EPI_ROW <= STAGE * 5 / 4 ? BM / 2 : BM / 4;
    constexpr int STG0 = EPI_PR * EPI_ROW > STAGE ? EPI_PR * EPI_ROW : STAGE;
    __shared__ __attribute__((aligned(16))) char stg0[DMA ? STG0 : 16];
    __shared__ __attribute__((aligned(16))) char stg1[DMA ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) char stg2[DMA && NBUF > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) char stg3[DMA && NBUF > 3 ? STAGE : 16];
    __shared__ float rs[BM];     // row scale (1/rms)
    __shared__ float qsum[(FLAGS & EPI_RMS_PARTS) ? BM * 16 : 1];  // per-quad sums of the RMS partials
    // EPI_UPDATE: the tile's k|v rows as stored (bf16), read by the fused step
    __shared__ __attribute__((aligned(16))) bf16 kvs[(FLAGS & EPI_UPDATE) ? BM * (BN + 8) : 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int grp = tid / NTG, gtid = tid % NTG, wave = gtid >> 6;
    char* const smem = KS == 1 ? smem_all : smem_all + grp * NBUF * STAGE;  // this K group's stage buffers
    auto stage_ptr = [&](int b) -> char* {
        if constexpr (DMA) return b == 0 ? stg0 : b == 1 ? stg1 : b == 2 ? stg2 : stg3;
        else return smem + b * STAGE;
    };
    const int wm = wave / WN, wn = wave % WN;
    const int gq = lane >> 5;
    const int64_t m0 = (int64_t)by * BM;
    const int n0 = bx * BN;
    // PAIRED: tile n holds rows n*BN/2 .. of W[0] (its left half) and of W[1] (its right half)
    constexpr bool PAIRED = (FLAGS & EPI_PAIRKV) != 0;
    constexpr int HB = BN / 2;
    const int seg = PAIRED ? 0 : n0 / g.seg_n;
    const int pcol = (n0 / BN) * HB;  // PAIRED: first column of this tile in each segment
    const int64_t ldw = g.ldw ? g.ldw : g.K;  // row stride of W
    const bf16* W = (const bf16*)g.W[seg] + k_off + (int64_t)(n0 % g.seg_n) * ldw;
    const bf16* A = (const bf16*)g.A + k_off;

    // this thread's chunks: slot s = NTG*i + gtid, tile row s/8, chunk column (s%8) ^ ((row/2)%8)
    const bf16* a_src[LA];
    int a_slot[LA];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int s = NTG * i + gtid, r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
        int64_t row = m0 + r;
        row = row < g.M ? row : g.M - 1;  // rows past M read a valid row; their results are dropped
        a_src[i] = A + row * g.lda + c * 8;
        a_slot[i] = s;
    }
    const bf16* w_src[LW];
#pragma unroll
    for (int i = 0; i < LW; ++i) {
        const int s = NTG * i + gtid, r = s >> 3, c = (s & 7) ^ ((r >> 1) & 7);
        w_src[i] = PAIRED ? (const bf16*)g.W[r >= HB] + k_off + (int64_t)(pcol + r % HB) * ldw + c * 8
                          : W + (int64_t)r * ldw + c * 8;
    }

    bf16x8 ra[DMA ? 1 : D][LA], rw[DMA ? 1 : D][LW];
    const int a_k = g.a_k ? g.a_k : g.K;  // A's own columns: column k reads k mod a_k (split weights)
    auto load = [&](int u, int k0) {
        const int ka = k0 >= a_k ? k0 - a_k : k0;
#pragma unroll
        for (int i = 0; i < LA; ++i) ra[u][i] = *reinterpret_cast<const bf16x8*>(a_src[i] + ka);
#pragma unroll
        for (int i = 0; i < LW; ++i) rw[u][i] = *reinterpret_cast<const bf16x8*>(w_src[i] + k0);
    };
    auto store = [&](int u, int buf) {
        char* base = smem + buf * STAGE;
#pragma unroll
        for (int i = 0; i < LA; ++i) *reinterpret_cast<bf16x8*>(base + a_slot[i] * 16) = ra[u][i];
#pragma unroll
        for (int i = 0; i < LW; ++i) *reinterpret_cast<bf16x8*>(base + (A_CH + NTG * i + gtid) * 16) = rw[u][i];
    };

    // PIPE_DMA: K tile k0 into LDS stage buf (a wave's 64 lanes fill 64 consecutive slots)
    auto dma = [&](int buf, int k0) {
        const int ka = k0 >= a_k ? k0 - a_k : k0;
        char* base = stage_ptr(buf) + wave * 64 * 16;
#pragma unroll
        for (int i = 0; i < LA; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + ka),
                                             (__attribute__((address_space(3))) void*)(base + NTG * i * 16), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < LW; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(w_src[i] + k0),
                                             (__attribute__((address_space(3))) void*)(base + (A_CH + NTG * i) * 16), 16,
                                             0, 0);
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < AE; ++e) acc[i][j][e] = 0.f;
    float ss[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) ss[i] = 0.f;

    // operand fetch: lane holds 8 consecutive k of row (lane % MF), k-group lane / MF
    const int lrow = lane % MF, lgrp = lane / MF;
    auto compute = [&](int buf) {
        const char* sA = stage_ptr(buf);
        const char* sW = sA + A_CH * 16;
        constexpr int KM = MF == 32 ? 16 : 32;  // k per MFMA
        constexpr int GPS = KM / 8;             // 16-byte chunks per MFMA k-slice
#pragma unroll
        for (int kk = 0; kk < BK / KM; ++kk) {
            const int c = GPS * kk + lgrp;
            bf16x8 aop[FM], wop[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * TMW + i * MF + lrow;
                aop[i] = *reinterpret_cast<const bf16x8*>(sA + swz(r, c) * 16);
                if ((FLAGS & EPI_RMS) && wn == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) ss[i] += (float)aop[i][e] * (float)aop[i][e];
                }
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int r = wn * TNW + j * MF + lrow;
                wop[j] = *reinterpret_cast<const bf16x8*>(sW + swz(r, c) * 16);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    if constexpr (MF == 32)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], wop[j], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[i], wop[j], acc[i][j], 0, 0, 0);
                }
        }
    };

    // The K loop is branch-free so that the compiler's wait counts stay exact
    // (the host guarantees (K/64/KS) % D == 0): prefetches past the last tile
    // reload the last tile, and the one spare store lands in the LDS buffer
    // nobody reads again. K group grp covers K tiles [grp*KT, (grp+1)*KT).
    const int KT = g.K / BK / KS;
    const int k_first = grp * KT * BK;
    const int last = k_first + (KT - 1) * BK;
    if constexpr (DMA) {
        // prologue: tiles 0..D-2 in flight into stages 0..D-2
#pragma unroll
        for (int u = 0; u < D - 1; ++u) dma(u, min(k_first + u * BK, last));
    } else {
        // prologue: tiles 0..D-1 in flight, tile 0 in LDS buffer 0, tile D replaces it in the ring
#pragma unroll
        for (int u = 0; u < D; ++u) load(u, min(k_first + u * BK, last));
        store(0, 0);
        load(0, min(k_first + D * BK, last));
    }
    // partial sums of squares of this tile's A rows (EPI_RMS_PARTS), laid out
    // [M][n_parts] with n_parts % 4 == 0 and <= 64: fetched as float4s behind
    // the first K tiles (so the main loop's first waits do not include them),
    // combined after the main loop.
    constexpr int PQ = (BM * 16 + NT - 1) / NT;  // float4 quads per thread
    float4 pss[(FLAGS & EPI_RMS_PARTS) ? PQ : 1];
    const int qpr = g.n_parts / 4;                // quads per row
    if (FLAGS & EPI_RMS_PARTS) {
        // unconditional loads (rows clamped into the tile and the matrix): a
        // conditional load would make the compiler wait for every load in
        // flight where the branches join; quads past the tile are dropped later
#pragma unroll
        for (int i = 0; i < PQ; ++i) {
            const int idx = tid + NT * i, r = min(idx / qpr, BM - 1);
            const int64_t row = min(m0 + r, g.M - 1);
            pss[i] = reinterpret_cast<const float4*>(g.rss_in + row * g.n_parts)[idx % qpr];
        }
    }

    constexpr int LDT = BN + 4;  // fp32 row pitch in LDS
    // rows per pass through the stage buffers (register staging: both stages, so a 128-row fp32
    // tile takes two passes, 256 rows four; PIPE_DMA: stage 0 alone); each K group stages its
    // partial tile in its own buffers
    constexpr int EPI_BYTES = DMA ? STG0 : 2 * STAGE;  // LDS the epilogue's fp32 tile passes may use
    constexpr int PR = (BM * LDT * 4 <= EPI_BYTES) ? BM : (BM / 2 * LDT * 4 <= EPI_BYTES) ? BM / 2 : (BM / 4 * LDT * 4 <= EPI_BYTES) ? BM / 4 : BM / 8;
    static_assert(PR * LDT * 4 <= EPI_BYTES && BM % PR == 0, "fp32 tile passes fit the stage buffers");
    constexpr int CPRW = BN / 8;               // 8-column runs per row
    constexpr int RUNS = (PR * CPRW + NT - 1) / NT;  // runs per thread per pass
    // The epilogue's run of a thread: (pass, it) -> tile row rl of the pass and
    // first column c0 (a run past the tile, when NT does not divide the run
    // count, is computed on row 0 and dropped: every lane takes part in the
    // shuffles of the epilogue).
    auto run_of = [&](int it, int& rl, int& c0) {
        const int xr = tid + NT * it;
        const int x = xr < PR * CPRW ? xr : xr % CPRW;
        rl = x / CPRW;
        c0 = (x % CPRW) * 8;
        return xr < PR * CPRW;
    };
    // Residual rows of the epilogue, when a thread has few runs: loaded now,
    // unconditionally (rows clamped into the matrix), so their latency hides
    // under the main loop.
    constexpr int NPASS = BM / PR;
    constexpr bool PREF_R = (FLAGS & EPI_RESID) && NPASS * RUNS <= 2;
    Raw8<TR> res_pre[PREF_R ? NPASS * RUNS : 1];
    if constexpr (PREF_R) {
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass)
#pragma unroll
            for (int it = 0; it < RUNS; ++it) {
                int rl, c0;
                run_of(it, rl, c0);
                const int64_t row = min(m0 + pass * PR + rl, g.M - 1);
                res_pre[pass * RUNS + it].load((const TR*)g.R + row * g.ldr + n0 + c0);
            }
    }

    if constexpr (DMA) {
        // iteration kt: this wave's loads of tile kt are complete once at most
        // the D-2 newer tiles' loads are outstanding (the row-sum and residual
        // loads above only make the first waits longer); the barrier then makes
        // every wave's part visible and frees stage (kt-1)%D, which takes tile
        // kt+D-1. Prefetches past the last tile reload it into stages nobody
        // reads again; they have landed before the epilogue reuses the stages.
        for (int kt0 = 0; kt0 < KT; kt0 += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                const int kt = kt0 + u;
                wait_vm<(D - 2) * (LA + LW)>();
                dma_barrier();
                dma((u + D - 1) % D, min(k_first + (kt + D - 1) * BK, last));
                compute(u);
            }
        }
        wait_vm<0>();
    } else {
        for (int kt0 = 0; kt0 < KT; kt0 += D) {
#pragma unroll
            for (int u = 0; u < D; ++u) {
                const int kt = kt0 + u;
                lds_barrier();                 // tile kt is in LDS; tile kt-1's buffer is free
                compute(kt & 1);
                const int nu = (u + 1) % D;    // ring stage of tile kt+1 (constant once unrolled)
                store(nu, (kt + 1) & 1);
                load(nu, min(k_first + (kt + 1 + D) * BK, last));
            }
        }
    }

    if (FLAGS & EPI_RMS_PARTS) {
        // each quad's sum to LDS, then one thread per row adds its row's quads
#pragma unroll
        for (int i = 0; i < PQ; ++i) {
            const int idx = tid + NT * i, r = idx / qpr;
            if (r < BM) qsum[r * 16 + idx % qpr] = (pss[i].x + pss[i].y) + (pss[i].z + pss[i].w);
        }
        __syncthreads();
        for (int r = tid; r < BM; r += NT) {
            float v = 0.f;
            for (int q = 0; q < qpr; ++q) v += qsum[r * 16 + q];
            rs[r] = g.no_rms ? 1.f : rsqrtf(v / (float)a_k + g.eps);
        }
    }
    if (FLAGS & EPI_RMS) {
        if (wn == 0) {
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                float s2 = ss[i];
#pragma unroll
                for (int x = MF; x < 64; x <<= 1) s2 += __shfl_xor(s2, x, 64);  // lanes sharing the row
                if (lgrp == 0) rs[wm * TMW + i * MF + lrow] = g.no_rms ? 1.f : rsqrtf(s2 / (float)g.K + g.eps);
            }
        }
    }
    // Epilogue. The fp32 tile goes through LDS (the free stage buffers) so that
    // each thread then owns runs of 8 consecutive columns of one row: 16-byte
    // stores and residual loads, and each 32-column group's sum of squares is a
    // 4-lane shuffle.
    static_assert(NT % CPRW == 0 && CPRW % 4 == 0, "runs map onto lanes evenly");
    static_assert(!(FLAGS & EPI_ROWSS) || (BN % kRowSSTile == 0 && CPRW >= 4), "32-column groups");
    float* tl = reinterpret_cast<float*>(DMA ? stg0 : smem);          // this group's partial tile
    const float* tl0 = reinterpret_cast<const float*>(DMA ? stg0 : smem_all);
    TC* C = (TC*)g.C[seg] + c_off;
#pragma unroll
    for (int pass = 0; pass < BM / PR; ++pass) {
    __syncthreads();  // the stage buffers are free (last reads done; rs ready; previous pass consumed)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < AE; ++e) {
                // accumulator layouts: 32x32 -> column lane%32, row 8*(e/4) + 4*(lane/32) + e%4;
                //                      16x16 -> column lane%16, row 4*(lane/16) + e
                const int r = wm * TMW + i * MF + (MF == 32 ? 8 * (e >> 2) + 4 * gq + (e & 3) : 4 * lgrp + e);
                const int c = wn * TNW + j * MF + lrow;
                if (r >= pass * PR && r < (pass + 1) * PR) tl[(r - pass * PR) * LDT + c] = acc[i][j][e];
            }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < RUNS; ++it) {
        int rl, c0;
        const bool in_tile = run_of(it, rl, c0);
        const int x = rl * CPRW + c0 / 8;  // run index within the pass (4 consecutive lanes per 32 columns)
        const int r = pass * PR + rl;
        const int64_t row = m0 + r;
        const bool ok = in_tile && row < g.M;
        const int col = n0 + c0;
        // column within the output segment
        const int ocol = PAIRED ? pcol + c0 % HB : col % g.seg_n;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kg = 0; kg < KS; ++kg) {
            const float* t = tl0 + kg * (NBUF * STAGE / 4) + rl * LDT + c0;
            const float4 p0 = *reinterpret_cast<const float4*>(t);
            const float4 p1 = *reinterpret_cast<const float4*>(t + 4);
            v[0] += p0.x; v[1] += p0.y; v[2] += p0.z; v[3] += p0.w;
            v[4] += p1.x; v[5] += p1.y; v[6] += p1.z; v[7] += p1.w;
        }
        if (FLAGS & (EPI_RMS | EPI_RMS_PARTS)) {
            const float sc = rs[r];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= sc;
        }
        if (FLAGS & EPI_GELU) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = gelu_erf(v[e]);
        }
        if constexpr ((FLAGS & EPI_DGELU) != 0) {
            if (ok) {
                float pre[8];
                load8((const TR*)g.R + row * g.ldr + col, pre);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] *= gelu_erf_grad(pre[e]);
            }
        }
        if constexpr ((FLAGS & EPI_QKNORM) != 0) {
            // per-head RMS (query/key norm): a head's head_dim/8 runs sit in as many
            // consecutive lanes (BN is a multiple of head_dim); seg is uniform per workgroup
            if ((g.qkn_mask >> (PAIRED ? (c0 >= HB) : seg)) & 1) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
                for (int o = 1; o < g.head_dim / 8; o <<= 1) ss += __shfl_xor(ss, o, 64);
                const float sc = rsqrtf(ss / (float)g.head_dim + g.eps);
                const float* gg = g.qkn_gain[PAIRED ? (c0 >= HB) : seg];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] *= sc * (gg ? gg[ocol + e] : 1.f);
            }
        }
        if constexpr (PREF_R) {
            const Raw8<TR>& res = res_pre[pass * RUNS + it];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = res[e] + g.rscale * v[e];
        } else if ((FLAGS & EPI_RESID) && ok) {
            float res[8];
            load8((const TR*)g.R + row * g.ldr + col, res);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = res[e] + g.rscale * v[e];
        }
        float stored[8];
        if (ok) {
            TC* dst = (PAIRED ? (TC*)g.C[c0 >= HB] + c_off : C) + row * g.ldc + ocol;
            if constexpr (sizeof(TC) == 2) {
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o[e] = (bf16)v[e];
                    stored[e] = (float)o[e];
                }
                *reinterpret_cast<bf16x8*>(dst) = o;
                if constexpr ((FLAGS & EPI_UPDATE) != 0)
                    *reinterpret_cast<bf16x8*>(&kvs[r * (BN + 8) + c0]) = o;
            } else {
                store8((float*)dst, v);
#pragma unroll
                for (int e = 0; e < 8; ++e) stored[e] = v[e];
            }
            if (FLAGS & EPI_COPY) {
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = (bf16)v[e];
                *reinterpret_cast<bf16x8*>((bf16*)g.C2 + row * g.ldc + ocol) = o;
            }
        }
        if (FLAGS & EPI_ROWSS) {
            // sum of squares of the stored values over this row's 32-column group:
            // the group's 4 runs sit in 4 consecutive lanes
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sq += ok ? stored[e] * stored[e] : 0.f;
            sq += __shfl_xor(sq, 1, 64);
            sq += __shfl_xor(sq, 2, 64);
            if (ok && (x % 4) == 0) g.rss_out[row * (g.N / kRowSSTile) + col / kRowSSTile] = sq;
        }
    }
    }
    if constexpr ((FLAGS & EPI_UPDATE) != 0) {
        static_assert((FLAGS & EPI_PAIRKV) && BN == 128 && sizeof(TC) == 2, "the fused step reads one head's k|v");
        __syncthreads();  // kvs complete
        fused_small_step(g.upd, kvs, BN + 8, m0, (int)min((int64_t)BM, g.M - m0), g.M, n0 / BN, tid, NT);
    }
}

template <typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN, int D, int MF, int KS = 1>
__global__ __launch_bounds__(64 * WM * WN * KS) void gemm_pipe_kernel(GemmArgs g) {
    gemm_pipe_body<TC, TR, FLAGS, BM, BN, WM, WN, D, MF, KS>(g, blockIdx.x, blockIdx.y);
}

// Several products of the same kind and shape in one launch (blockIdx.z picks
// the product; row counts may differ, the grid covers the largest): the
// per-position products of the layers of a stack, which one at a time leave
// most of the chip idle.
struct GemmGroup {
    GemmArgs g[kMaxGemmGroup];
};
static_assert(sizeof(GemmGroup) <= 3584, "kernel argument size");

template <typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN, int D, int MF, int KS = 1>
__global__ __launch_bounds__(64 * WM * WN * KS) void gemm_pipe_group_kernel(GemmGroup gg) {
    uint32_t bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    if constexpr ((FLAGS & PIPE_XCD) != 0) {
        // workgroup i runs on XCD i % 8: give XCD x the x-th eighth of the (z, y, x) tiles
        const uint32_t gxy = gridDim.x * gridDim.y, nwg = gxy * gridDim.z;
        uint32_t lin = bx + gridDim.x * (by + gridDim.y * bz);
        if ((nwg & 7) == 0) lin = (lin & 7) * (nwg >> 3) + (lin >> 3);
        bz = lin / gxy;
        by = (lin % gxy) / gridDim.x;
        bx = lin % gridDim.x;
    }
    const GemmArgs& g = gg.g[bz];
    if ((int64_t)by * BM >= g.M) return;  // past this product's rows (the whole workgroup)
    gemm_pipe_body<TC, TR, FLAGS, BM, BN, WM, WN, D, MF, KS>(g, bx, by);
}

// Products that differ only in their K range, one per blockIdx.z (a weight
// gradient's reduction over rows split into ranges, each writing its own
// partial): product z reads A and W from column z * k_step on and writes C
// from element z * c_step on.
struct GemmSplitK {
    GemmArgs g;  // product 0
    int64_t k_step, c_step;
};
static_assert(sizeof(GemmSplitK) <= 3584, "kernel argument size");

template <typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN, int D, int MF>
__global__ __launch_bounds__(64 * WM * WN) void gemm_pipe_splitk_kernel(GemmSplitK sk) {
    const int64_t z = blockIdx.z;
    gemm_pipe_body<TC, TR, FLAGS, BM, BN, WM, WN, D, MF, 1>(sk.g, blockIdx.x, blockIdx.y, z * sk.k_step,
                                                            z * sk.c_step);
}

template <typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN, int D, int MF = 32>
static hipError_t run_splitk(const GemmSplitK& sk, int splits, hipStream_t s) {
    const int64_t row_tiles = (sk.g.M + BM - 1) / BM;
    if (row_tiles > 65535 || splits > 65535) return hipErrorInvalidConfiguration;
    dim3 grid((uint32_t)(sk.g.N / BN), (uint32_t)row_tiles, (uint32_t)splits);
    hipLaunchKernelGGL((gemm_pipe_splitk_kernel<TC, TR, FLAGS, BM, BN, WM, WN, D, MF>), grid, dim3(64 * WM * WN), 0,
                       s, sk);
    return hipGetLastError();
}

// The products of one launch: n argument sets of one kind and shape (n <= kMaxGemmGroup).
struct GemmSet {
    const GemmArgs* g;
    int n;
    int64_t max_m;
};

template <typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN, int D, int MF = 32, int KS = 1>
static hipError_t run_pipe(const GemmSet& gs, hipStream_t s) {
    const GemmArgs& g = gs.g[0];
    const int64_t row_tiles = (gs.max_m + BM - 1) / BM;
    if (row_tiles > 65535) return hipErrorInvalidConfiguration;  // grid y limit
    if (gs.n == 1) {
        dim3 grid((uint32_t)(g.N / BN), (uint32_t)row_tiles);
        hipLaunchKernelGGL((gemm_pipe_kernel<TC, TR, FLAGS, BM, BN, WM, WN, D, MF, KS>), grid,
                           dim3(64 * WM * WN * KS), 0, s, g);
    } else {
        GemmGroup gg{};
        for (int i = 0; i < gs.n; ++i) gg.g[i] = gs.g[i];
        dim3 grid((uint32_t)(g.N / BN), (uint32_t)row_tiles, (uint32_t)gs.n);
        hipLaunchKernelGGL((gemm_pipe_group_kernel<TC, TR, FLAGS, BM, BN, WM, WN, D, MF, KS>), grid,
                           dim3(64 * WM * WN * KS), 0, s, gg);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- fp32 SIMT

template <typename TR, int FLAGS>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= g.M * (int64_t)g.N) return;
    const int64_t row = idx / g.N;
    const int col = (int)(idx % g.N);
    const int seg = col / g.seg_n;
    const float* a = (const float*)g.A + row * g.lda;
    const float* w = (const float*)g.W[seg] + (int64_t)(col % g.seg_n) * (g.ldw ? g.ldw : g.K);
    float acc = 0.f, ss = 0.f;
    for (int k = 0; k < g.K; ++k) {
        acc += a[k] * w[k];
        if (FLAGS & EPI_RMS) ss += a[k] * a[k];
    }
    const float rstd = ((FLAGS & EPI_RMS) && !g.no_rms) ? rsqrtf(ss / (float)g.K + g.eps) : 1.f;
    epilogue_store<FLAGS, TR, float>(g, (float*)g.C[seg], row, col, acc, rstd);
}

template <typename TR, int FLAGS>
static hipError_t run_f32(const GemmArgs& g, hipStream_t s) {
    const int64_t n = g.M * (int64_t)g.N;
    hipLaunchKernelGGL((gemm_f32_kernel<TR, FLAGS>), dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, g);
    return hipGetLastError();
}

// ---------------------------------------------------------------- dispatch

bool gemm_shape_supported(rt_dtype dt, int64_t M, int N, int K) {
    if (M <= 0 || N <= 0 || K <= 0) return false;
    if (dt == RT_F32) return true;
    return (K % 64 == 0) && (N % 128 == 0);
}

template <int D, int KS>
static hipError_t dispatch_bf16(GemmKind kind, const GemmSet& gs, hipStream_t s) {
    const GemmArgs& g = gs.g[0];  // the shape and flags every product of the set shares
    const bool big = gs.max_m >= 4096;
    const bool grouped = !big && gs.n >= 2;
    // 256-column tiles need whole tiles inside every output segment (a 128-wide
    // remainder takes the 128x128 tiles)
    const bool wide = g.N % 256 == 0 && g.seg_n % 256 == 0;
    const bool tall = big && wide;
    // at most 16 rows (a small batch, a decode step): 16-row tiles, 32 columns
    // wide, K split over 2 or 4 wave groups (M = 8: W_o 4.3 us against 5.9 with
    // the 64-row tiles, W_1 4.6 against 7.6, W_2 8.2 against 12.2, W_kv 4.3
    // against 6.4; with many more, narrower workgroups streaming the weights)
    const bool skinny = gs.max_m <= 16 && gs.n == 1;
    // Tiles measured on MI355X at the per-position shapes (M = batch = 512): small
    // 64-row tiles of 16x16x32 MFMAs (four independent accumulators per wave),
    // with K split over 2 or 4 wave groups where that measured faster (W_2,
    // W_o, W_kv); products over N*B rows (the up-front projection, every
    // product of the Transformer layer, the backward's batched products) use
    // 256x256 tiles with the K tiles loaded straight into two LDS stages
    // (128x128 where an output segment is not whole 256-column tiles).
    // Several per-position products in one launch
    // (the layers of a stack) fill the chip, and larger tiles then win: for six
    // products of 512 rows, W_1 128x128 (four waves side by side, 128x32 each)
    // 44.8 us against 58.8 with the per-position tile (48.3 with 2x2 waves),
    // W_2 128x128 with 2 K groups 44.3 against 77.4, W_o 64x64 18.9 against
    // 25.6, W_kv 128x128 25.3 against 38.6. Then W_kv 128x256 with eight waves
    // 22.9 / 25.6 against 24.9 / 28.0 for 128x128 (two boxes; eight side by
    // side 23.7 against 24.5 for 2x4), W_o's 64x64 prefetching 2 K tiles 18.2
    // against 19.3 with 4, W_2's K groups of four waves stacked (32x128 each)
    // 47.4 against 50.2 for 2x2 (a slow box); 256-row or 256-column tiles
    // measured slower for W_1 (50.5-58.2) and W_2 (60.0-63.1). Eight waves per
    // 128x128 tile (half the accumulators and prefetch registers per wave, twice
    // the waves hiding the loads): W_1 4x2 waves (32x64 each, 128 VGPRs) 44.0
    // against 56.4 for 1x4, W_2 2x4 waves without a K split (112 VGPRs) 40.9
    // against 46.8 for two K groups of 4x1 (one box).
    switch (kind) {
        case GemmKind::QKV:
            if constexpr (KS == 1) {
                // tall (N*B-row) products prefetch 2 K tiles: at 1M rows x 3072 x 1024 the
                // partial-sum variant measured 535 us per 65536 rows with 2, 806 with 4
                if (g.rss_in) {  // row sums of squares given (row_sumsq): RMS from the partials
                    if (g.qkn_mask)
                        return big ? run_pipe<bf16, float, EPI_RMS_PARTS | EPI_QKNORM, 128, 128, 2, 2, 2, 32>(gs, s)
                                   : run_pipe<bf16, float, EPI_RMS_PARTS | EPI_QKNORM, 64, 64, 2, 2, D, 16>(gs, s);
                    // tall products (N*B rows, and a stack's chunks of 65536): 256x256 tiles, eight
                    // waves of 128x64, K tiles straight into two LDS stages: 601 us per chunk against
                    // 702 for 128x128 with four waves side by side, 7.85 ms at 1M rows against 9.05
                    // for 2x2 waves (256x256 with register staging spills)
                    if (tall) return run_pipe<bf16, float, EPI_RMS_PARTS | PIPE_DMA, 256, 256, 2, 4, 2, 32>(gs, s);
                    return big ? run_pipe<bf16, float, EPI_RMS_PARTS, 128, 128, 2, 2, 2, 32>(gs, s)
                               : run_pipe<bf16, float, EPI_RMS_PARTS, 64, 64, 2, 2, D, 16>(gs, s);
                }
                if (g.qkn_mask)
                    return big ? run_pipe<bf16, float, EPI_RMS | EPI_QKNORM, 128, 128, 2, 2, 2, 32>(gs, s)
                               : run_pipe<bf16, float, EPI_RMS | EPI_QKNORM, 64, 64, 2, 2, D, 16>(gs, s);
                return big ? run_pipe<bf16, float, EPI_RMS, 128, 128, 2, 2, 2, 32>(gs, s)
                           : run_pipe<bf16, float, EPI_RMS, 64, 64, 2, 2, D, 16>(gs, s);
            }
            break;
        case GemmKind::WO:  // h (fp32) and its bf16 copy, plus partial sums of h^2 for the MLP's RMS
            if constexpr (KS <= 4) {
                if (skinny) return run_pipe<float, bf16, EPI_RESID | EPI_COPY | EPI_ROWSS, 16, 32, 1, 1, D, 16, KS>(gs, s);
            }
            if constexpr (KS == 1) {
                // every tall product (N*B rows) takes the 256x256 direct-to-LDS tiles the tall
                // q|k'|v' projection uses: a Transformer layer's forward at B=512 drops 3-4%
                // (19.7 against 20.6 ms at N=1024), the RT layer's backward 0.5%
                if (tall) return run_pipe<float, bf16, EPI_RESID | EPI_COPY | EPI_ROWSS | PIPE_DMA, 256, 256, 2, 4, 2, 32>(gs, s);
                if (big) return run_pipe<float, bf16, EPI_RESID | EPI_COPY | EPI_ROWSS, 128, 128, 2, 2, 2, 32>(gs, s);
                if (grouped) {
                    // K tiles straight into a 4-stage LDS ring, XCD-grouped tiles: 17.4 us against 19.3
                    if constexpr (D == 4)
                        return run_pipe<float, bf16, EPI_RESID | EPI_COPY | EPI_ROWSS | PIPE_DMA | PIPE_XCD, 64, 64, 2, 2, 4,
                                        16>(gs, s);
                    return run_pipe<float, bf16, EPI_RESID | EPI_COPY | EPI_ROWSS, 64, 64, 2, 2, 2, 16>(gs, s);
                }
            }
            if constexpr (KS <= 2)
                if (!big)  // 2x2 waves per K group (6.6 us against 7.0 for 2x1, M = 512)
                    return run_pipe<float, bf16, EPI_RESID | EPI_COPY | EPI_ROWSS, 64, kRowSSTile, 2, 2, D, 16, KS>(gs, s);
            break;
        case GemmKind::W1:
            if constexpr (KS <= 4) {
                if (skinny) return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_GELU, 16, 32, 1, 1, D, 16, KS>(gs, s);
            }
            if constexpr (KS == 1) {
                if (grouped) return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_GELU, 128, 128, 4, 2, 2, 32>(gs, s);
                // one layer's per-position product: 128x64 with eight waves of 32x32
                // (11.4 us against 13.1 for 64x64 with four waves, M = 512)
                if (tall) return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_GELU | PIPE_DMA, 256, 256, 2, 4, 2, 32>(gs, s);
                return big ? run_pipe<bf16, float, EPI_RMS_PARTS | EPI_GELU, 128, 128, 2, 2, 2, 32>(gs, s)
                           : run_pipe<bf16, float, EPI_RMS_PARTS | EPI_GELU, 128, 64, 4, 2, 2, 32>(gs, s);
            }
            break;
        case GemmKind::W2:  // z, plus partial sums of z^2 (as stored) for the persistent pair's RMS
            if constexpr (KS <= 4) {
                if (skinny) return run_pipe<bf16, float, EPI_RESID | EPI_ROWSS, 16, 32, 1, 1, D, 16, KS>(gs, s);
            }
            if constexpr (KS == 1) {
                if (tall) return run_pipe<bf16, float, EPI_RESID | EPI_ROWSS | PIPE_DMA, 256, 256, 2, 4, 2, 32>(gs, s);
                if (big) return run_pipe<bf16, float, EPI_RESID | EPI_ROWSS, 128, 128, 2, 2, 2, 32>(gs, s);
                if (grouped) {
                    // K tiles straight into a 4-stage LDS ring, XCD-grouped tiles: 40.4-40.8 us against
                    // 44.9-45.1 (the weight and A fetches from outside L2 halve: 66 MB against 126)
                    if constexpr (D == 4)
                        return run_pipe<bf16, float, EPI_RESID | EPI_ROWSS | PIPE_DMA | PIPE_XCD, 128, 128, 2, 4, 4, 32>(
                            gs, s);
                    return run_pipe<bf16, float, EPI_RESID | EPI_ROWSS, 128, 128, 2, 4, 2, 32>(gs, s);
                }
            }
            if (!big) return run_pipe<bf16, float, EPI_RESID | EPI_ROWSS, 64, kRowSSTile, 2, 1, D, 16, KS>(gs, s);
            break;
        case GemmKind::KV_UPDATE:
            if constexpr (KS <= 2) {
                if (g.qkn_mask)
                    return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_PAIRKV | EPI_UPDATE | EPI_QKNORM, 32, 128, 1, 4, D,
                                    16, KS>(gs, s);
                return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_PAIRKV | EPI_UPDATE, 32, 128, 1, 4, D, 16, KS>(gs, s);
            }
            break;
        case GemmKind::KV:
            if constexpr (KS <= 4) {
                if (skinny) {  // the query/key norm needs a head's columns in one tile
                    if (g.qkn_mask) return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_QKNORM, 16, 64, 1, 2, D, 16, KS>(gs, s);
                    return run_pipe<bf16, float, EPI_RMS_PARTS, 16, 32, 1, 1, D, 16, KS>(gs, s);
                }
            }
            if constexpr (KS == 1) {
                if (grouped) {
                    if (g.qkn_mask) return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_QKNORM, 128, 128, 2, 2, 2, 32>(gs, s);
                    // 256 columns (sixteen waves of 32x64, 23.3 us against 25.6 for eight side by side)
                    // where no tile straddles the k|v boundary
                    if (g.seg_n % 256 == 0) return run_pipe<bf16, float, EPI_RMS_PARTS, 128, 256, 4, 4, 2, 32>(gs, s);
                    return run_pipe<bf16, float, EPI_RMS_PARTS, 128, 128, 2, 2, 2, 32>(gs, s);
                }
            }
            if constexpr (KS <= 2) {
                if (g.qkn_mask) return run_pipe<bf16, float, EPI_RMS_PARTS | EPI_QKNORM, 64, 64, 2, 2, D, 16, KS>(gs, s);
                return run_pipe<bf16, float, EPI_RMS_PARTS, 64, 64, 2, 2, D, 16, KS>(gs, s);
            }
            break;
        case GemmKind::W1_PRE:
            if constexpr (KS == 1) {
                if (tall) return run_pipe<bf16, float, EPI_RMS_PARTS | PIPE_DMA, 256, 256, 2, 4, 2, 32>(gs, s);
                return big ? run_pipe<bf16, float, EPI_RMS_PARTS, 128, 128, 2, 2, 2, 32>(gs, s)
                           : run_pipe<bf16, float, EPI_RMS_PARTS, 64, 64, 2, 2, D, 16>(gs, s);
            }
            break;
        case GemmKind::W2_BWD:
            if constexpr (KS == 1) {  // 128x64 with eight waves: 11.1 us against 12.0 for 64x64 (M = 512)
                if (!big) return run_pipe<bf16, bf16, EPI_DGELU, 128, 64, 4, 2, 2, 32>(gs, s);
            }
            if (!big) return run_pipe<bf16, bf16, EPI_DGELU, 64, 64, 2, 2, D, 16, KS>(gs, s);
            break;
        case GemmKind::PLAIN:
            if constexpr (KS == 1) {
                if (tall) return run_pipe<float, float, PIPE_DMA, 256, 256, 2, 4, 2, 32>(gs, s);
                if (big) return run_pipe<float, float, 0, 128, 128, 2, 2, 2, 32>(gs, s);
            }
            // per-position adjoint products (M = 512, N = 1024): 64x32 tiles, twice the
            // workgroups of 64x64 (K = 1024: 6.1 against 6.9 us, 2048: 8.6 against 9.9,
            // 4096: 14.1 against 17.6)
            if constexpr (KS <= 2) {  // 2x2 waves per K group: 5.6 / 8.0 us against 6.1 / 8.7 (K = 1024 / 2048)
                if (!big) return run_pipe<float, float, 0, 64, 32, 2, 2, D, 16, KS>(gs, s);
            }
            if (!big) return run_pipe<float, float, 0, 64, 32, 2, 1, D, 16, KS>(gs, s);
            break;
        case GemmKind::WGRAD:  // the K ranges of a weight gradient: launch_gemm_splitk
            break;
    }
    return hipErrorInvalidValue;
}

// K groups per workgroup for a kind and shape: the measured choice when K
// divides into an even number of 64-wide tiles per group, else fewer.
static int k_groups(GemmKind kind, const GemmArgs& g, int64_t max_m, int n) {
    if (max_m >= 4096) return 1;
    int ks = kind == GemmKind::W2 ? 4
             : (kind == GemmKind::WO || kind == GemmKind::KV || kind == GemmKind::KV_UPDATE) ? 2
             : kind == GemmKind::PLAIN ? (g.K >= 4096 ? 4 : 2) : 1;  // W2_BWD: 12.1 us against 13.1 with 2
    if (n >= 2 && kind != GemmKind::KV_UPDATE) ks = 1;  // several products per launch (eight-wave tiles)
    if (n == 1 && max_m <= 16 && (kind == GemmKind::WO || kind == GemmKind::W1 || kind == GemmKind::W2 ||
                                  kind == GemmKind::KV))
        ks = kind == GemmKind::W2 ? 4 : 2;  // at most 16 rows
    const int kt = g.K / 64;
    while (ks > 1 && !(kt % ks == 0 && (kt / ks) % 2 == 0)) ks /= 2;
    return ks;
}

// fp32 layers: per-head RMS of the stored segments in place (query/key norm),
// one thread per (row, head).
__global__ __launch_bounds__(256) void qk_norm_f32_kernel(float* C, int64_t M, int ldc, int seg_n, int head_dim,
                                                           const float* gain, float eps) {
    const int heads = seg_n / head_dim;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * heads) return;
    float* x = C + (idx / heads) * ldc + (idx % heads) * head_dim;
    const float* gg = gain ? gain + (idx % heads) * head_dim : nullptr;
    float ss = 0.f;
    for (int i = 0; i < head_dim; ++i) ss += x[i] * x[i];
    const float sc = rsqrtf(ss / (float)head_dim + eps);
    for (int i = 0; i < head_dim; ++i) x[i] *= sc * (gg ? gg[i] : 1.f);
}

static hipError_t qk_norm_f32(const GemmArgs& g, hipStream_t s) {
    for (int seg = 0; seg < 3; ++seg) {
        if (!((g.qkn_mask >> seg) & 1)) continue;
        const int64_t n = g.M * (g.seg_n / g.head_dim);
        hipLaunchKernelGGL(qk_norm_f32_kernel, dim3((uint32_t)((n + 255) / 256)), dim3(256), 0, s, (float*)g.C[seg],
                           g.M, (int)g.ldc, g.seg_n, g.head_dim, g.qkn_gain[seg], g.eps);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

static hipError_t launch_gemm_f32(GemmKind kind, const GemmArgs& g, hipStream_t s) {
    hipError_t e = hipErrorInvalidValue;
    switch (kind) {
        case GemmKind::QKV: e = run_f32<float, EPI_RMS>(g, s); break;
        case GemmKind::WO: e = run_f32<float, EPI_RESID>(g, s); break;
        case GemmKind::W1: e = run_f32<float, EPI_RMS | EPI_GELU>(g, s); break;
        case GemmKind::W2: e = run_f32<float, EPI_RESID>(g, s); break;
        case GemmKind::KV: e = run_f32<float, EPI_RMS>(g, s); break;
        case GemmKind::KV_UPDATE: return hipErrorInvalidValue;  // bf16 layers only
        case GemmKind::W1_PRE: e = run_f32<float, EPI_RMS>(g, s); break;
        case GemmKind::PLAIN: e = run_f32<float, 0>(g, s); break;
        case GemmKind::W2_BWD: e = run_f32<float, EPI_DGELU>(g, s); break;
        case GemmKind::WGRAD: e = run_f32<float, 0>(g, s); break;
    }
    if (e != hipSuccess || !g.qkn_mask) return e;
    return qk_norm_f32(g, s);
}

// Products that may share a launch: the same shape and the same epilogue inputs.
static bool same_shape(const GemmArgs& a, const GemmArgs& b) {
    return a.N == b.N && a.K == b.K && a.a_k == b.a_k && a.ldw == b.ldw && a.no_rms == b.no_rms && a.seg_n == b.seg_n &&
           a.n_parts == b.n_parts &&
           (a.rss_in != nullptr) == (b.rss_in != nullptr) && a.qkn_mask == b.qkn_mask &&
           a.head_dim == b.head_dim && a.M > 0 && b.M > 0;
}

hipError_t launch_gemm(rt_dtype dt, GemmKind kind, const GemmArgs& g, hipStream_t s) {
    return launch_gemm_group(dt, kind, &g, 1, s);
}

hipError_t launch_gemm_group(rt_dtype dt, GemmKind kind, const GemmArgs* gs, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    for (int i = 1; i < n; ++i)
        if (!same_shape(gs[0], gs[i])) return hipErrorInvalidValue;
    if (dt == RT_F32) {  // one launch per product
        for (int i = 0; i < n; ++i) {
            const hipError_t e = launch_gemm_f32(kind, gs[i], s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    // K is a multiple of 128 (an even number of 64-wide K tiles); each K group
    // prefetches 4 tiles ahead when its tile count divides by 4, else 2
    if ((gs[0].K / 64) % 2) return hipErrorInvalidValue;
    for (int i0 = 0; i0 < n; i0 += kMaxGemmGroup) {
        GemmSet set{gs + i0, n - i0 < kMaxGemmGroup ? n - i0 : kMaxGemmGroup, 0};
        for (int i = 0; i < set.n; ++i) set.max_m = set.g[i].M > set.max_m ? set.g[i].M : set.max_m;
        const int ks = k_groups(kind, set.g[0], set.max_m, set.n);
        const bool d4 = (set.g[0].K / 64 / ks) % 4 == 0;
        hipError_t e = hipErrorInvalidValue;
        switch (ks) {
            case 1: e = d4 ? dispatch_bf16<4, 1>(kind, set, s) : dispatch_bf16<2, 1>(kind, set, s); break;
            case 2: e = d4 ? dispatch_bf16<4, 2>(kind, set, s) : dispatch_bf16<2, 2>(kind, set, s); break;
            case 4: e = d4 ? dispatch_bf16<4, 4>(kind, set, s) : dispatch_bf16<2, 4>(kind, set, s); break;
        }
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemm_splitk(rt_dtype dt, GemmKind kind, const GemmArgs& g, int splits, int64_t k_step,
                              int64_t c_step, hipStream_t s) {
    if (kind != GemmKind::WGRAD || splits <= 0 || g.M <= 0) return hipErrorInvalidValue;
    if (dt == RT_F32) {  // one launch per K range
        for (int z = 0; z < splits; ++z) {
            GemmArgs a = g;
            a.A = (const float*)g.A + z * k_step;
            a.W[0] = (const float*)g.W[0] + z * k_step;
            a.C[0] = (float*)g.C[0] + z * c_step;
            const hipError_t e = launch_gemm_f32(kind, a, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    if ((g.K / 64) % 2 || g.N % 128 || g.seg_n != g.N) return hipErrorInvalidValue;
    const GemmSplitK sk{g, k_step, c_step};
    // K of 10^4..10^5 rows per range. 256x256 tiles with two LDS stages, eight waves of 128x64 (the
    // tall products' tile): at d = 1024, F = 4096 and 16 ranges a d x d gradient is 256 workgroups,
    // a d x F one 1024. Else 128x128 with eight waves of 32x64, the K tiles straight into a 4-stage
    // LDS ring where the range divides into 4-tile groups.
    if (g.N % 256 == 0 && g.M >= 256) return run_splitk<float, float, PIPE_DMA, 256, 256, 2, 4, 2, 32>(sk, splits, s);
    if ((g.K / 64) % 4 == 0) return run_splitk<float, float, PIPE_DMA, 128, 128, 4, 2, 4, 32>(sk, splits, s);
    return run_splitk<float, float, 0, 128, 128, 4, 2, 2, 32>(sk, splits, s);
}

// ---------------------------------------------------------------- row sums of squares

// out[row][q] = sum of x[row][c]^2 over the q-th quarter of the row's columns
// (one wave per row, 8 columns per lane and step; D % 32 == 0): the RMS
// partials a product reads with EPI_RMS_PARTS instead of summing its own A
// rows inside its K loop.
template <typename T>
__global__ __launch_bounds__(64) void row_sumsq_kernel(const T* x, int D, float* out) {
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    const int quarter = D / 4;
    float ss[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane * 8; c < D; c += 512) {
        float v[8];
        load8(x + row * D + c, v);
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a += v[e] * v[e];
        const int qi = c / quarter;  // 8 columns never straddle a quarter (quarter % 8 == 0)
#pragma unroll
        for (int q = 0; q < 4; ++q) ss[q] += q == qi ? a : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
        for (int o = 32; o > 0; o >>= 1) ss[q] += __shfl_xor(ss[q], o, 64);
    if (lane == 0) *reinterpret_cast<float4*>(out + row * 4) = make_float4(ss[0], ss[1], ss[2], ss[3]);
}

hipError_t launch_row_sumsq(rt_dtype dt, const void* x, int64_t rows, int D, float* out, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (rows >= (1LL << 26) || D % 32) return hipErrorInvalidConfiguration;
    if (dt == RT_BF16)
        hipLaunchKernelGGL(row_sumsq_kernel<bf16>, dim3((uint32_t)rows), dim3(64), 0, s, (const bf16*)x, D, out);
    else
        hipLaunchKernelGGL(row_sumsq_kernel<float>, dim3((uint32_t)rows), dim3(64), 0, s, (const float*)x, D, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------- gain folding

__global__ __launch_bounds__(256) void fold_gain_f32_kernel(const float* W, const float* g, float* out, int64_t rows,
                                                             int cols) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * cols) return;
    out[idx] = W[idx] * g[idx % cols];
}

// bf16: the product W g (exact in fp32 up to one rounding) as a rounded bf16
// value and the bf16 of what that rounding dropped, in the two halves of the row.
__global__ __launch_bounds__(256) void fold_gain_bf16_kernel(const bf16* W, const float* g, bf16* out, int64_t rows,
                                                             int cols) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * cols) return;
    const int64_t r = idx / cols;
    const int c = (int)(idx % cols);
    const float p = (float)W[idx] * g[c];
    const bf16 hi = (bf16)p;
    out[r * 2 * cols + c] = hi;
    out[r * 2 * cols + cols + c] = (bf16)(p - (float)hi);
}

hipError_t launch_fold_gain(rt_dtype dt, const void* W, const float* g, void* W_out, int64_t rows, int cols,
                            hipStream_t s) {
    const int64_t n = rows * cols;
    const dim3 grid((uint32_t)((n + 255) / 256));
    if (dt == RT_BF16)
        hipLaunchKernelGGL(fold_gain_bf16_kernel, grid, dim3(256), 0, s, (const bf16*)W, g, (bf16*)W_out, rows, cols);
    else
        hipLaunchKernelGGL(fold_gain_f32_kernel, grid, dim3(256), 0, s, (const float*)W, g, (float*)W_out, rows, cols);
    return hipGetLastError();
}

}  // namespace rt
