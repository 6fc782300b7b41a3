// Projection GEMMs of the RT layer: C = epilogue(A * W^T), W row-major [out][in].
//
// Reading note (lshu.cn/news/403416), translated paper section 2: every
// projection acts on an RMS-normalised vector. RMS(a) * W^T equals
// rstd(a) * (a * W^T) row by row, so the normalisation is fused: the kernel
// accumulates sum(a^2) of its A rows while staging them (each workgroup
// streams whole rows, K is never split) and scales the product in the
// epilogue. Section 2.1: the MLP is W_2 GELU(W_1 .) and both branches are
// added to the residual stream, also fused here.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 on gfx950, fp32 accumulation; tiles
// staged global -> registers -> LDS with the next K tile prefetched into
// registers while the current one is multiplied. fp32 path: plain SIMT,
// one thread per output (used by small fp32 layers).
#include "rt_device.h"
#include "rt_internal.h"

namespace rt {

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

template <int FLAGS, typename TR, typename TC>
__device__ __forceinline__ void epilogue_store(const GemmArgs& g, TC* C, int64_t row, int64_t col, float v,
                                               float rstd) {
    if (FLAGS & EPI_RMS) v *= rstd;
    if (FLAGS & EPI_GELU) v = gelu_erf(v);
    if (FLAGS & EPI_RESID) v = to_f32(((const TR*)g.R)[row * g.ldr + col]) + g.rscale * v;
    C[row * g.ldc + (col % g.seg_n)] = from_f32<TC>(v);
}

// ---------------------------------------------------------------- bf16 MFMA

template <typename TA, typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmArgs g) {
    constexpr int NT = 64 * WM * WN;
    constexpr int BK = 64;
    constexpr int LDS_STRIDE = BK + 8;          // bf16 elements per LDS row (16 B pad)
    constexpr int TMW = BM / WM, TNW = BN / WN;  // wave tile
    constexpr int FM = TMW / 32, FN = TNW / 32;
    constexpr int CA = BM * (BK / 8) / NT;       // 8-element A chunks per thread
    constexpr int CW = BN * (BK / 8) / NT;
    static_assert(CA >= 1 && CW >= 1 && FM >= 1 && FN >= 1, "tile too small for the workgroup");
    static_assert(BM * (BK / 8) % NT == 0 && BN * (BK / 8) % NT == 0, "chunks must divide evenly");

    __shared__ bf16 As[BM * LDS_STRIDE];
    __shared__ bf16 Ws[BN * LDS_STRIDE];
    __shared__ float rs[BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int seg = n0 / g.seg_n;
    const bf16* W = (const bf16*)g.W[seg] + (int64_t)(n0 % g.seg_n) * g.K;
    const TA* A = (const TA*)g.A;

    const int crow = tid / (BK / 8);  // first row this thread stages
    const int ck = (tid % (BK / 8)) * 8;
    constexpr int ROWS_PER_PASS = NT / (BK / 8);

    bf16x8 ra[CA], rw[CW];
    float ss[CA];
#pragma unroll
    for (int r = 0; r < CA; ++r) ss[r] = 0.f;

    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int r = 0; r < CA; ++r) {
            const int64_t row = m0 + crow + r * ROWS_PER_PASS;
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (row < g.M) load8(A + row * g.lda + k0 + ck, v);
            if (FLAGS & EPI_RMS) {
#pragma unroll
                for (int e = 0; e < 8; ++e) ss[r] += v[e] * v[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) ra[r][e] = (bf16)v[e];
        }
#pragma unroll
        for (int r = 0; r < CW; ++r) {
            const int row = crow + r * ROWS_PER_PASS;
            rw[r] = *reinterpret_cast<const bf16x8*>(W + (int64_t)row * g.K + k0 + ck);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int KT = g.K / BK;
    load_tiles(0);
    for (int kt = 0; kt < KT; ++kt) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < CA; ++r)
            *reinterpret_cast<bf16x8*>(&As[(crow + r * ROWS_PER_PASS) * LDS_STRIDE + ck]) = ra[r];
#pragma unroll
        for (int r = 0; r < CW; ++r)
            *reinterpret_cast<bf16x8*>(&Ws[(crow + r * ROWS_PER_PASS) * LDS_STRIDE + ck]) = rw[r];
        __syncthreads();
        if (kt + 1 < KT) load_tiles((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int kofs = kk * 16 + (lane >> 5) * 8;
            bf16x8 aop[FM], wop[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                aop[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * TMW + i * 32 + (lane & 31)) * LDS_STRIDE + kofs]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                wop[j] = *reinterpret_cast<const bf16x8*>(&Ws[(wn * TNW + j * 32 + (lane & 31)) * LDS_STRIDE + kofs]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop[i], wop[j], acc[i][j], 0, 0, 0);
        }
    }

    if (FLAGS & EPI_RMS) {
#pragma unroll
        for (int r = 0; r < CA; ++r) {
            const float s = group_sum<BK / 8>(ss[r]);
            if ((tid % (BK / 8)) == 0) rs[crow + r * ROWS_PER_PASS] = rsqrtf(s / (float)g.K + g.eps);
        }
        __syncthreads();
    }

    TC* C = (TC*)g.C[seg];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                // 32x32 accumulator layout: lane holds column lane%32, rows 8*(e/4) + 4*(lane/32) + e%4
                const int r = wm * TMW + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int c = wn * TNW + j * 32 + (lane & 31);
                const int64_t row = m0 + r;
                if (row < g.M) epilogue_store<FLAGS, TR, TC>(g, C, row, n0 + c, acc[i][j][e], (FLAGS & EPI_RMS) ? rs[r] : 1.f);
            }
}

template <typename TA, typename TC, typename TR, int FLAGS, int BM, int BN, int WM, int WN>
static hipError_t run_bf16(const GemmArgs& g, hipStream_t s) {
    dim3 grid((uint32_t)(g.N / BN), (uint32_t)((g.M + BM - 1) / BM));
    hipLaunchKernelGGL((gemm_bf16_kernel<TA, TC, TR, FLAGS, BM, BN, WM, WN>), grid, dim3(64 * WM * WN), 0, s, g);
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
    const float* w = (const float*)g.W[seg] + (int64_t)(col % g.seg_n) * g.K;
    float acc = 0.f, ss = 0.f;
    for (int k = 0; k < g.K; ++k) {
        acc += a[k] * w[k];
        if (FLAGS & EPI_RMS) ss += a[k] * a[k];
    }
    const float rstd = (FLAGS & EPI_RMS) ? rsqrtf(ss / (float)g.K + g.eps) : 1.f;
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
    return (K % 64 == 0) && (N % 64 == 0);
}

hipError_t launch_gemm(rt_dtype dt, GemmKind kind, const GemmArgs& g, hipStream_t s) {
    if (dt == RT_F32) {
        switch (kind) {
            case GemmKind::QKV: return run_f32<float, EPI_RMS>(g, s);
            case GemmKind::WO: return run_f32<float, EPI_RESID>(g, s);
            case GemmKind::W1: return run_f32<float, EPI_RMS | EPI_GELU>(g, s);
            case GemmKind::W2: return run_f32<float, EPI_RESID>(g, s);
            case GemmKind::KV: return run_f32<float, EPI_RMS>(g, s);
        }
        return hipErrorInvalidValue;
    }
    const bool big = g.M >= 4096;
    switch (kind) {
        case GemmKind::QKV:
            return big ? run_bf16<bf16, bf16, float, EPI_RMS, 128, 128, 2, 2>(g, s)
                       : run_bf16<bf16, bf16, float, EPI_RMS, 64, 64, 2, 2>(g, s);
        case GemmKind::WO: return run_bf16<bf16, float, bf16, EPI_RESID, 64, 64, 2, 2>(g, s);
        case GemmKind::W1: return run_bf16<float, bf16, float, EPI_RMS | EPI_GELU, 64, 64, 2, 2>(g, s);
        case GemmKind::W2: return run_bf16<bf16, bf16, float, EPI_RESID, 64, 64, 2, 2>(g, s);
        case GemmKind::KV: return run_bf16<bf16, bf16, float, EPI_RMS, 64, 64, 2, 2>(g, s);
    }
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- gain folding

template <typename T>
__global__ __launch_bounds__(256) void fold_gain_kernel(const T* W, const float* g, T* out, int64_t rows, int cols) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * cols) return;
    out[idx] = from_f32<T>(to_f32(W[idx]) * g[idx % cols]);
}

hipError_t launch_fold_gain(rt_dtype dt, const void* W, const float* g, void* W_out, int64_t rows, int cols,
                            hipStream_t s) {
    const int64_t n = rows * cols;
    const dim3 grid((uint32_t)((n + 255) / 256));
    if (dt == RT_BF16)
        hipLaunchKernelGGL(fold_gain_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)W, g, (bf16*)W_out, rows, cols);
    else
        hipLaunchKernelGGL(fold_gain_kernel<float>, grid, dim3(256), 0, s, (const float*)W, g, (float*)W_out, rows,
                           cols);
    return hipGetLastError();
}

}  // namespace rt
