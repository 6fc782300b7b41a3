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
#include <cstdint>
#include <type_traits>

#include "rt_device.h"
#include "rt_internal.h"

namespace rt {

namespace {

template <typename T>
__device__ __forceinline__ float ld1(const T* p) { return (float)*p; }

template <typename T>
__device__ __forceinline__ T cvt(float v) { return (T)v; }

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

__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// One wave per row, 8 consecutive columns per lane and step (D % 8 == 0): the
// adjoint of x for y = g x / r given y_bar,
//   out = base + g y_bar / r - x sum(g y_bar x) / (D r^3),
// and optionally out2 = scale2 * out in TO, rinv_out[row] = 1 / r.
template <typename TX, typename TO>
__global__ __launch_bounds__(64) void rms_bwd_kernel(const TX* x, const float* ybar, const float* g, float eps,
                                                     const float* base, float* out, TO* out2, float scale2,
                                                     float* rinv_out, int D) {
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    const TX* xr = x + row * D;
    const float* yr = ybar + row * D;
    float ss = 0.f, sg = 0.f;
    for (int c = lane * 8; c < D; c += 512) {
        float xv[8], yv[8];
        load8(xr + c, xv);
        load8(yr + c, yv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ss += xv[e] * xv[e];
            sg += (g ? g[c + e] : 1.f) * yv[e] * xv[e];
        }
    }
    ss = wave_sum(ss);
    sg = wave_sum(sg);
    const float rinv = rsqrtf(ss / (float)D + eps);
    const float coef = sg * rinv * rinv * rinv / (float)D;
    for (int c = lane * 8; c < D; c += 512) {
        float xv[8], yv[8], bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, o[8];
        load8(xr + c, xv);
        load8(yr + c, yv);
        if (base) load8(base + row * D + c, bv);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = bv[e] + (g ? g[c + e] : 1.f) * yv[e] * rinv - xv[e] * coef;
        store8(out + row * D + c, o);
        if (out2) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= scale2;
            store8(out2 + row * D + c, o);
        }
    }
    if (rinv_out && lane == 0) rinv_out[row] = rinv;
}

// One wave per row: out = g x / r in TO (the normalised input of a product).
template <typename TX, typename TO>
__global__ __launch_bounds__(64) void rms_apply_kernel(const TX* x, const float* g, float eps, TO* out, int D) {
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x;
    const TX* xr = x + row * D;
    float ss = 0.f;
    for (int c = lane * 8; c < D; c += 512) {
        float xv[8];
        load8(xr + c, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += xv[e] * xv[e];
    }
    const float rinv = rsqrtf(wave_sum(ss) / (float)D + eps);
    for (int c = lane * 8; c < D; c += 512) {
        float xv[8];
        load8(xr + c, xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) xv[e] *= (g ? g[c + e] : 1.f) * rinv;
        store8(out + row * D + c, xv);
    }
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

// Second level: part2[g][c] = sum of part[blk][c] over the blocks of group g
// (groups of kGainGroup blocks, in block order).
__global__ __launch_bounds__(256) void gain_fold_kernel(const float* part, int64_t nblk, int D, float* part2) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= D) return;
    const int64_t b0 = (int64_t)blockIdx.y * kGainGroup;
    const int64_t b1 = b0 + kGainGroup < nblk ? b0 + kGainGroup : nblk;
    float acc = 0.f;
    for (int64_t b = b0; b < b1; ++b) acc += part[b * D + c];
    part2[(int64_t)blockIdx.y * D + c] = acc;
}

// Last level: out[c] (+)= sum over groups of part2[g][c], in group order.
__global__ __launch_bounds__(256) void gain_sum_kernel(const float* part2, int ngroups, int D, float* out,
                                                       int accumulate) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= D) return;
    float acc = 0.f;
    for (int g = 0; g < ngroups; ++g) acc += part2[(int64_t)g * D + c];
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
    if (rows >= (1LL << 26) || D % 8) return hipErrorInvalidConfiguration;  // rows * 64 work-items < 2^32
    const dim3 grid((uint32_t)rows), block(64);
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
    if (rows >= (1LL << 26) || D % 8) return hipErrorInvalidConfiguration;  // rows * 64 work-items < 2^32
    const dim3 grid((uint32_t)rows), block(64);
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

int64_t gain_grad_blocks(int64_t rows) {
    const int64_t nblk = (rows + kGainRowsPerBlock - 1) / kGainRowsPerBlock;
    return nblk + (nblk + kGainGroup - 1) / kGainGroup;  // first-level blocks + second-level groups
}

hipError_t launch_gain_grad(rt_dtype x_dt, const float* ybar, const void* x, const float* rinv, int64_t rows, int D,
                            float* part, float* out, int accumulate, hipStream_t s) {
    const int64_t nblk = (rows + kGainRowsPerBlock - 1) / kGainRowsPerBlock;
    if (nblk <= 0 || nblk >= (1LL << 24)) return nblk <= 0 ? hipSuccess : hipErrorInvalidConfiguration;
    if (x_dt == RT_BF16)
        hipLaunchKernelGGL(gain_part_kernel<bf16>, dim3((uint32_t)nblk), dim3(256), 0, s, ybar, (const bf16*)x, rinv,
                           rows, D, kGainRowsPerBlock, part);
    else
        hipLaunchKernelGGL(gain_part_kernel<float>, dim3((uint32_t)nblk), dim3(256), 0, s, ybar, (const float*)x,
                           rinv, rows, D, kGainRowsPerBlock, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ngroups = (nblk + kGainGroup - 1) / kGainGroup;
    float* part2 = part + nblk * D;  // (the caller's buffer holds both levels)
    hipLaunchKernelGGL(gain_fold_kernel, dim3((uint32_t)((D + 255) / 256), (uint32_t)ngroups), dim3(256), 0, s, part,
                       nblk, D, part2);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gain_sum_kernel, dim3((uint32_t)((D + 255) / 256)), dim3(256), 0, s, part2, (int)ngroups, D,
                       out, accumulate);
    return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(zero_f32_kernel, grid_for(n), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

// ------------------------------------------------------------- weight gradients
//
// W_bar[o][i] (+)= sum_r A_bar[r][o] U[r][i] over R = N*B rows. The reduction
// runs along the rows of both operands, so both are transposed first into
// row-major [O][Rp] and [I][Rp] copies (zero past row R, Rp a multiple of the
// split), and the product C = A_bar^T U^T^T is the library's MFMA GEMM with
// K = Rp, split into up to kWgradSplits K ranges run as one launch (blockIdx.z
// picks the range; at O = I = 1024 a product has 16 output tiles of 256x256,
// so 16 ranges give 256 workgroups), each writing its own fp32 partial; a last
// pass adds the partials (and the previous gradient when accumulating) in a
// fixed order.

namespace {

// dst[c][r] = r < rows ? src[r * lds + c] : 0 for c < cols, r < rows_pad
// (64x64 tiles through LDS; a thread moves 4 consecutive elements each way).
template <typename T>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const T* src, int64_t rows, int64_t lds, int cols,
                                                            T* dst, int64_t rows_pad) {
    __shared__ T tile[64][64 + 4];
    const int64_t r0 = (int64_t)blockIdx.y * 64;
    const int c0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int q = tid + 256 * it, rl = q >> 4, cl = (q & 15) * 4;  // row, first column of the quad
        const int64_t r = r0 + rl;
        const int c = c0 + cl;
        T v[4] = {T(0.f), T(0.f), T(0.f), T(0.f)};
        if (r < rows && c < cols) {  // cols % 4 == 0: a quad is all in or all out
            const T* p = src + r * lds + c;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = p[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[rl][cl + e] = v[e];
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int q = tid + 256 * it, cl = q >> 4, rl = (q & 15) * 4;  // destination row (column of src), 4 rows
        const int c = c0 + cl;
        if (c >= cols) continue;
        T* p = dst + (int64_t)c * rows_pad + r0 + rl;
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = tile[rl + e][cl];
    }
}

// The same for bf16 with 16-byte accesses both ways: a thread loads 8 columns
// of a source row, and stores 8 consecutive source rows of one column (cols,
// lds and rows_pad multiples of 8, both pointers 16-byte aligned; the tile's
// LDS rows padded by 8 elements stay 16-byte aligned).
__global__ __launch_bounds__(256) void transpose_pad_bf16x8_kernel(const bf16* src, int64_t rows, int64_t lds,
                                                                   int cols, bf16* dst, int64_t rows_pad) {
    constexpr int PITCH = 64 + 8;
    __shared__ __attribute__((aligned(16))) bf16 tile[64 * PITCH];
    const int64_t r0 = (int64_t)blockIdx.y * 64;
    const int c0 = blockIdx.x * 64;
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int q = tid + 256 * it, rl = q >> 3, ch = (q & 7) * 8;  // tile row, first column of the run
        const int64_t r = r0 + rl;
        const int c = c0 + ch;
        bf16x8 v;
        if (r < rows && c < cols) {
            v = *reinterpret_cast<const bf16x8*>(src + r * lds + c);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (bf16)0.f;
        }
        *reinterpret_cast<bf16x8*>(&tile[rl * PITCH + ch]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int q = tid + 256 * it, cl = q >> 3, rr = (q & 7) * 8;  // destination row, first of 8 source rows
        const int c = c0 + cl;
        if (c >= cols) continue;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[(rr + e) * PITCH + cl];
        *reinterpret_cast<bf16x8*>(dst + (int64_t)c * rows_pad + r0 + rr) = v;
    }
}

// out[i] = (accumulate ? out[i] : 0) + sum_s part[s][i], s in order (n % 4 == 0).
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float* part, int splits, int64_t n, float* out,
                                                           int accumulate) {
    for (int64_t q = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; q < n; q += (int64_t)gridDim.x * 256 * 4) {
        float4 acc = accumulate ? *reinterpret_cast<const float4*>(out + q) : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int sp = 0; sp < splits; ++sp) {
            const float4 v = *reinterpret_cast<const float4*>(part + sp * n + q);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        *reinterpret_cast<float4*>(out + q) = acc;
    }
}

template <typename T>
hipError_t transpose_pad(const void* src, int64_t rows, int64_t lds, int cols, void* dst, int64_t rows_pad,
                         hipStream_t s) {
    if (cols % 4 || rows_pad % 64 || rows_pad / 64 > 65535) return hipErrorInvalidValue;
    const dim3 grid((uint32_t)((cols + 63) / 64), (uint32_t)(rows_pad / 64));
    if (std::is_same<T, bf16>::value && cols % 8 == 0 && lds % 8 == 0 && (uintptr_t)src % 16 == 0 &&
        (uintptr_t)dst % 16 == 0)
        hipLaunchKernelGGL(transpose_pad_bf16x8_kernel, grid, dim3(256), 0, s, (const bf16*)src, rows, lds, cols,
                           (bf16*)dst, rows_pad);
    else
        hipLaunchKernelGGL(transpose_pad_kernel<T>, grid, dim3(256), 0, s, (const T*)src, rows, lds, cols, (T*)dst,
                           rows_pad);
    return hipGetLastError();
}

}  // namespace

WgradPlan wgrad_plan(int64_t rows) {
    WgradPlan p{};
    p.splits = rows >= (int64_t)kWgradSplits * 1024 ? kWgradSplits : 1;
    const int64_t unit = 128 * (int64_t)p.splits;  // every split's K an even number of 64-wide tiles
    p.rows_pad = (rows + unit - 1) / unit * unit;
    return p;
}

hipError_t weight_grad(rt_dtype dt, const void* abar, int64_t lda, const void* u, int64_t ldu, int64_t R, int O,
                       int I, float* out, bool accumulate, bool u_ready, const WgradScratch& ws, hipStream_t s) {
    const WgradPlan pl = wgrad_plan(R);
    if (pl.rows_pad != ws.rows_pad || O % 4 || I % 4) return hipErrorInvalidValue;
    hipError_t e = dt == RT_BF16 ? transpose_pad<bf16>(abar, R, lda, O, ws.ta, pl.rows_pad, s)
                                 : transpose_pad<float>(abar, R, lda, O, ws.ta, pl.rows_pad, s);
    if (e != hipSuccess) return e;
    if (!u_ready) {  // U^T is already in ws.tu from the previous call with the same U
        e = dt == RT_BF16 ? transpose_pad<bf16>(u, R, ldu, I, ws.tu, pl.rows_pad, s)
                          : transpose_pad<float>(u, R, ldu, I, ws.tu, pl.rows_pad, s);
        if (e != hipSuccess) return e;
    }
    const int64_t kc = pl.rows_pad / pl.splits;
    GemmArgs a{};  // K range 0; range sp starts sp * kc columns on and writes partial sp
    a.A = ws.ta; a.lda = pl.rows_pad;
    a.W[0] = ws.tu; a.ldw = pl.rows_pad;
    a.C[0] = ws.part; a.ldc = I; a.seg_n = I;
    a.M = O; a.N = I; a.K = (int32_t)kc;
    e = launch_gemm_splitk(dt, GemmKind::WGRAD, a, pl.splits, kc, (int64_t)O * I, s);
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)O * I;
    const int64_t blocks = (n / 4 + 255) / 256;
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((uint32_t)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                       ws.part, pl.splits, n, out, accumulate ? 1 : 0);
    return hipGetLastError();
}

}  // namespace rt
