// Bandwidth probes for the benchmark (not part of the layer's path): what the
// GPU's HBM sustains for plain streaming work with the update kernels' mix of
// traffic, so that each kernel's bandwidth can be put beside it.
//   rt_probe_stream(n, r): out = a_1 ^ ... ^ a_r over n 16-byte elements per
//     tensor: r streams read, one written (r = 3: the blocked update's ~3:1
//     read:write mix; r = 1: a copy).
// Each thread moves 16-byte vectors, UNROLL independent loads in flight, over
// a grid-stride loop sized to fill every CU several times.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int UNROLL = 4;

template <int R>
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ a0, const uint4* __restrict__ a1,
                                                     const uint4* __restrict__ a2, uint4* __restrict__ out,
                                                     int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + (UNROLL - 1) * stride < n; i += UNROLL * stride) {
        uint4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            v[u] = a0[i + u * stride];
            if (R >= 2) {
                const uint4 w = a1[i + u * stride];
                v[u].x ^= w.x; v[u].y ^= w.y; v[u].z ^= w.z; v[u].w ^= w.w;
            }
            if (R >= 3) {
                const uint4 w = a2[i + u * stride];
                v[u].x ^= w.x; v[u].y ^= w.y; v[u].z ^= w.z; v[u].w ^= w.w;
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) out[i + u * stride] = v[u];
    }
    for (; i < n; i += stride) {
        uint4 v = a0[i];
        if (R >= 2) {
            const uint4 w = a1[i];
            v.x ^= w.x; v.y ^= w.y; v.z ^= w.z; v.w ^= w.w;
        }
        if (R >= 3) {
            const uint4 w = a2[i];
            v.x ^= w.x; v.y ^= w.y; v.z ^= w.z; v.w ^= w.w;
        }
        out[i] = v;
    }
}

}  // namespace

extern "C" {

// reads: 1..3 source tensors (a1, a2 unused below that); n16: 16-byte elements per tensor;
// blocks: grid size (0: 2048). Returns a hipError_t code.
int rt_probe_stream(const void* a0, const void* a1, const void* a2, void* out, int64_t n16, int reads, int blocks,
                    hipStream_t s) {
    if (!a0 || !out || n16 <= 0 || reads < 1 || reads > 3 || (reads >= 2 && !a1) || (reads >= 3 && !a2))
        return (int)hipErrorInvalidValue;
    const dim3 grid((uint32_t)(blocks > 0 ? blocks : 2048)), block(256);
    const uint4 *p0 = (const uint4*)a0, *p1 = (const uint4*)a1, *p2 = (const uint4*)a2;
    uint4* o = (uint4*)out;
    if (reads == 1) hipLaunchKernelGGL(stream_kernel<1>, grid, block, 0, s, p0, p1, p2, o, n16);
    else if (reads == 2) hipLaunchKernelGGL(stream_kernel<2>, grid, block, 0, s, p0, p1, p2, o, n16);
    else hipLaunchKernelGGL(stream_kernel<3>, grid, block, 0, s, p0, p1, p2, o, n16);
    return (int)hipGetLastError();
}

}
