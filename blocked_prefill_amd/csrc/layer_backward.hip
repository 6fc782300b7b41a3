// Kernels of the RT layer's backward pass beyond the attention map's gradient:
// weight transposes, adjoint packing, the RMS normalisation's adjoint, the
// GELU derivative, and the batched weight gradients.
//
// The layer (Recurrent Transformer reading note, lshu.cn/news/403416,
// translated paper sections 2.1-2.2) is differentiated by the chain rule; the
// pages state only that the backward can be batched outside the position loop
// (translated paper section 6.1; section 6.4 is a heading without a body).
// The per-position adjoint chain runs in abi.hip; this file holds its pieces.
//
// RMS(x) = g x / r with r = sqrt(mean(x^2) + eps) has the adjoint
//   x_bar = g y_bar / r - x sum(g y_bar x) / (d r^3),   g_bar += y_bar x / r.
// The GELU's derivative Phi(u) + u phi(u) is applied in the W_2^T product's
// epilogue (gemm.hip).
#include <rocblas/rocblas.h>

#include "rt_device.h"
#include "rt_internal.h"

namespace rt {

namespace {

template <typename T>
__device__ __forceinline__ float ld1(const T* p) { return (float)*p; }

template <typename T>
__device__ __forceinline__ T cvt(float v) { return (T)v; }

// Sum over a 256-thread workgroup (4 waves); every thread gets the result.
__device__ __forceinline__ float block_sum256(float v, float* red) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();  // red is free (a previous call's readers are done)
    if (lane == 0) red[wave] = v;
    __syncthreads();
    return red[0] + red[1] + red[2] + red[3];
}

// dst[c][col0 + r] = src[r][c] for src [rows][cols] (32x32 tiles through LDS).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* src, int64_t rows, int64_t cols, T* dst, int64_t ldd,
                                                        int64_t col0) {
    __shared__ T tile[32][33];
    const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int i = ty; i < 32; i += 8) {
        const int64_t r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) tile[i][tx] = src[r * cols + c];
    }
    __syncthreads();
    for (int i = ty; i < 32; i += 8) {
        const int64_t c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) dst[c * ldd + col0 + r] = tile[tx][i];
    }
}

// dst[r][s*D + c] = scale * src_s[r][c] for s < nsrc (fp32 sources, dst in T);
// one thread per 4 consecutive elements (D % 4 == 0).
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(T* dst, int64_t ldd, const float* s0, const float* s1,
                                                   const float* s2, int nsrc, int64_t rows, int D, float scale) {
    const int64_t per_row = (int64_t)nsrc * (D / 4);
    // quad index over rows * nsrc * D/4, grid-stride
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < rows * per_row; q += (int64_t)gridDim.x * 256) {
    const int64_t r = q / per_row;
    const int rem = (int)(q % per_row);
    const int s = rem / (D / 4), c = (rem % (D / 4)) * 4;
    const float* src = s == 0 ? s0 : (s == 1 ? s1 : s2);
    const float4 v = *reinterpret_cast<const float4*>(src + r * D + c);
    T* o = dst + r * ldd + (int64_t)s * D + c;
    o[0] = cvt<T>(scale * v.x);
    o[1] = cvt<T>(scale * v.y);
    o[2] = cvt<T>(scale * v.z);
    o[3] = cvt<T>(scale * v.w);
    }
}

// One workgroup per row: the adjoint of x for y = g x / r given y_bar,
//   out = base + g y_bar / r - x sum(g y_bar x) / (D r^3),
// and optionally out2 = scale2 * out in T, rinv_out[row] = 1 / r.
template <typename TX, typename TO>
__global__ __launch_bounds__(256) void rms_bwd_kernel(const TX* x, const float* ybar, const float* g, float eps,
                                                      const float* base, float* out, TO* out2, float scale2,
                                                      float* rinv_out, int D) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const TX* xr = x + row * D;
    const float* yr = ybar + row * D;
    float ss = 0.f, sg = 0.f;
    for (int c = threadIdx.x; c < D; c += 256) {
        const float xv = ld1(xr + c), gv = g ? g[c] : 1.f;
        ss += xv * xv;
        sg += gv * yr[c] * xv;
    }
    ss = block_sum256(ss, red);
    sg = block_sum256(sg, red);
    const float rinv = rsqrtf(ss / (float)D + eps);
    const float coef = sg * rinv * rinv * rinv / (float)D;
    for (int c = threadIdx.x; c < D; c += 256) {
        const float xv = ld1(xr + c), gv = g ? g[c] : 1.f;
        const float o = (base ? base[row * D + c] : 0.f) + gv * yr[c] * rinv - xv * coef;
        out[row * D + c] = o;
        if (out2) out2[row * D + c] = cvt<TO>(scale2 * o);
    }
    if (rinv_out && threadIdx.x == 0) rinv_out[row] = rinv;
}

// One workgroup per row: out = g x / r in T (the normalised input of a product).
template <typename TX, typename TO>
__global__ __launch_bounds__(256) void rms_apply_kernel(const TX* x, const float* g, float eps, TO* out, int D) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const TX* xr = x + row * D;
    float ss = 0.f;
    for (int c = threadIdx.x; c < D; c += 256) {
        const float xv = ld1(xr + c);
        ss += xv * xv;
    }
    ss = block_sum256(ss, red);
    const float rinv = rsqrtf(ss / (float)D + eps);
    for (int c = threadIdx.x; c < D; c += 256) out[row * D + c] = cvt<TO>((g ? g[c] : 1.f) * ld1(xr + c) * rinv);
}

// u = GELU(u) in place.
template <typename T>
__global__ __launch_bounds__(256) void gelu_inplace_kernel(T* u, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const float v = ld1(u + i);
        u[i] = cvt<T>(0.5f * v * (1.0f + erff(v * 0.70710678118654752f)));
    }
}

// Gain gradient, first level: part[blk][c] = sum over the block's rows of y_bar * x * rinv.
template <typename TX>
__global__ __launch_bounds__(256) void gain_part_kernel(const float* ybar, const TX* x, const float* rinv,
                                                        int64_t rows, int D, int rows_per_block, float* part) {
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
    for (int c = threadIdx.x; c < D; c += 256) {
        float acc = 0.f;
        for (int64_t r = r0; r < r1; ++r) acc += ybar[r * D + c] * ld1(x + r * D + c) * rinv[r];
        part[(int64_t)blockIdx.x * D + c] = acc;
    }
}

// Second level: out[c] (+)= sum over blocks of part[blk][c], in block order.
__global__ __launch_bounds__(256) void gain_sum_kernel(const float* part, int nblk, int D, float* out, int accumulate) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= D) return;
    float acc = 0.f;
    for (int b = 0; b < nblk; ++b) acc += part[(int64_t)b * D + c];
    out[c] = accumulate ? out[c] + acc : acc;
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// Grid of a grid-stride elementwise kernel over n items: at most 2^20
// workgroups (a launch's work-items must stay below 2^32).
dim3 grid_for(int64_t n) {
    const int64_t blocks = (n + 255) / 256;
    return dim3((uint32_t)(blocks < (1 << 20) ? blocks : (1 << 20)));
}

}  // namespace

hipError_t launch_transpose(rt_dtype dt, const void* src, int64_t rows, int64_t cols, void* dst, int64_t ldd,
                            int64_t col0, hipStream_t s) {
    const dim3 grid((uint32_t)((cols + 31) / 32), (uint32_t)((rows + 31) / 32));
    if (grid.y > 65535) return hipErrorInvalidConfiguration;
    if (dt == RT_BF16)
        hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)src, rows, cols, (bf16*)dst,
                           ldd, col0);
    else
        hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, s, (const float*)src, rows, cols, (float*)dst,
                           ldd, col0);
    return hipGetLastError();
}

hipError_t launch_pack(rt_dtype dt, void* dst, int64_t ldd, const float* s0, const float* s1, const float* s2,
                       int nsrc, int64_t rows, int D, float scale, hipStream_t s) {
    if (D % 4) return hipErrorInvalidValue;
    const int64_t n = rows * nsrc * (D / 4);
    if (n <= 0) return hipSuccess;
    if (dt == RT_BF16)
        hipLaunchKernelGGL(pack_kernel<bf16>, grid_for(n), dim3(256), 0, s, (bf16*)dst, ldd, s0, s1, s2, nsrc, rows,
                           D, scale);
    else
        hipLaunchKernelGGL(pack_kernel<float>, grid_for(n), dim3(256), 0, s, (float*)dst, ldd, s0, s1, s2, nsrc,
                           rows, D, scale);
    return hipGetLastError();
}

hipError_t launch_rms_bwd(rt_dtype x_dt, rt_dtype out2_dt, const void* x, const float* ybar, const float* g,
                          float eps, const float* base, float* out, void* out2, float scale2, float* rinv_out,
                          int64_t rows, int D, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (rows >= (1LL << 24)) return hipErrorInvalidConfiguration;  // rows * 256 work-items < 2^32
    const dim3 grid((uint32_t)rows), block(256);
    if (x_dt == RT_BF16 && out2_dt == RT_BF16)
        hipLaunchKernelGGL((rms_bwd_kernel<bf16, bf16>), grid, block, 0, s, (const bf16*)x, ybar, g, eps, base, out,
                           (bf16*)out2, scale2, rinv_out, D);
    else if (x_dt == RT_F32 && out2_dt == RT_BF16)
        hipLaunchKernelGGL((rms_bwd_kernel<float, bf16>), grid, block, 0, s, (const float*)x, ybar, g, eps, base, out,
                           (bf16*)out2, scale2, rinv_out, D);
    else if (x_dt == RT_BF16)
        hipLaunchKernelGGL((rms_bwd_kernel<bf16, float>), grid, block, 0, s, (const bf16*)x, ybar, g, eps, base, out,
                           (float*)out2, scale2, rinv_out, D);
    else
        hipLaunchKernelGGL((rms_bwd_kernel<float, float>), grid, block, 0, s, (const float*)x, ybar, g, eps, base,
                           out, (float*)out2, scale2, rinv_out, D);
    return hipGetLastError();
}

hipError_t launch_rms_apply(rt_dtype x_dt, rt_dtype out_dt, const void* x, const float* g, float eps, void* out,
                            int64_t rows, int D, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (rows >= (1LL << 24)) return hipErrorInvalidConfiguration;  // rows * 256 work-items < 2^32
    const dim3 grid((uint32_t)rows), block(256);
    if (x_dt == RT_BF16 && out_dt == RT_BF16)
        hipLaunchKernelGGL((rms_apply_kernel<bf16, bf16>), grid, block, 0, s, (const bf16*)x, g, eps, (bf16*)out, D);
    else if (x_dt == RT_F32 && out_dt == RT_BF16)
        hipLaunchKernelGGL((rms_apply_kernel<float, bf16>), grid, block, 0, s, (const float*)x, g, eps, (bf16*)out, D);
    else if (x_dt == RT_BF16)
        hipLaunchKernelGGL((rms_apply_kernel<bf16, float>), grid, block, 0, s, (const bf16*)x, g, eps, (float*)out, D);
    else
        hipLaunchKernelGGL((rms_apply_kernel<float, float>), grid, block, 0, s, (const float*)x, g, eps, (float*)out,
                           D);
    return hipGetLastError();
}

hipError_t launch_gelu_inplace(rt_dtype dt, void* u, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    if (dt == RT_BF16)
        hipLaunchKernelGGL(gelu_inplace_kernel<bf16>, grid_for(n), dim3(256), 0, s, (bf16*)u, n);
    else
        hipLaunchKernelGGL(gelu_inplace_kernel<float>, grid_for(n), dim3(256), 0, s, (float*)u, n);
    return hipGetLastError();
}

int64_t gain_grad_blocks(int64_t rows) { return (rows + kGainRowsPerBlock - 1) / kGainRowsPerBlock; }

hipError_t launch_gain_grad(rt_dtype x_dt, const float* ybar, const void* x, const float* rinv, int64_t rows, int D,
                            float* part, float* out, int accumulate, hipStream_t s) {
    const int64_t nblk = gain_grad_blocks(rows);
    if (nblk <= 0 || nblk >= (1LL << 24)) return nblk <= 0 ? hipSuccess : hipErrorInvalidConfiguration;
    if (x_dt == RT_BF16)
        hipLaunchKernelGGL(gain_part_kernel<bf16>, dim3((uint32_t)nblk), dim3(256), 0, s, ybar, (const bf16*)x, rinv,
                           rows, D, kGainRowsPerBlock, part);
    else
        hipLaunchKernelGGL(gain_part_kernel<float>, dim3((uint32_t)nblk), dim3(256), 0, s, ybar, (const float*)x,
                           rinv, rows, D, kGainRowsPerBlock, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gain_sum_kernel, dim3((uint32_t)((D + 255) / 256)), dim3(256), 0, s, part, (int)nblk, D, out,
                       accumulate);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_f32_kernel, grid_for(n), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

// ------------------------------------------------------------- weight gradients
//
// W_bar[o][i] (+)= sum_r A_bar[r][o] U[r][i] over R rows (a plain GEMM with the
// reduction over positions x batch rows), on rocBLAS: in column-major terms
// W_bar^T (I x O) = U^T (I x R) * A_bar (R x O).

namespace {
rocblas_handle g_blas[64];  // one handle per device, created on first use
}

hipError_t weight_grad(rt_dtype dt, const void* abar, int64_t lda, const void* u, int64_t ldu, int64_t R, int O,
                       int I, float* out, bool accumulate, hipStream_t s) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (R > 0x7fffffffLL || lda > 0x7fffffffLL || ldu > 0x7fffffffLL) return hipErrorInvalidValue;
    if (!g_blas[dev] && rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
        g_blas[dev] = nullptr;
        return hipErrorUnknown;
    }
    if (rocblas_set_stream(g_blas[dev], s) != rocblas_status_success) return hipErrorUnknown;
    const float alpha = 1.f, beta = accumulate ? 1.f : 0.f;
    const rocblas_datatype ab = dt == RT_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
    const rocblas_status st =
        rocblas_gemm_ex(g_blas[dev], rocblas_operation_none, rocblas_operation_transpose, I, O, (rocblas_int)R, &alpha,
                        u, ab, (rocblas_int)ldu, abar, ab, (rocblas_int)lda, &beta, out, rocblas_datatype_f32_r, I,
                        out, rocblas_datatype_f32_r, I, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
    return st == rocblas_status_success ? hipSuccess : hipErrorUnknown;
}

}  // namespace rt
