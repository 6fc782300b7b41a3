// rt_layer_decode_step_static: the decode step of rt_layer_decode_step for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation). Its scratch is a
// file-scope device array of a fixed size instead of a caller's workspace;
// every device that loads the library holds one copy of it until the process
// ends. The kernels are those of rt_layer_decode_step: the array's device
// address (taken once per device with hipGetSymbolAddress) is passed where
// that entry point passes the workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rt_internal.h"

// The array itself. In host code its name is a host-side stand-in, not a
// device address: host code uses only the address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[RT_DECODE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once taken

// The calling thread's current device's copy of the array (its address taken on
// the first call on that device, with that device current).
rt_status device_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return rt::set_error(RT_ERR_HIP, "hipGetDevice failed: ", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return rt::set_error(RT_ERR_UNSUPPORTED, "device index out of range", "");
    std::lock_guard<std::mutex> hold(g_lock);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return rt::set_error(RT_ERR_HIP, "hipGetSymbolAddress(scratch) failed: ", hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return RT_OK;
}

}  // namespace

extern "C" rt_status rt_layer_decode_step_static(const rt_layer_desc* desc, const rt_layer_weights* w,
                                                 int32_t n_past, const void* x_t, void* z_t, void* k_cache,
                                                 void* v_cache, rt_stream_t stream) {
    const rt_status ok = rt::check_decode_args(desc, w, n_past, x_t, z_t, k_cache, v_cache);  // no HIP call
    if (ok != RT_OK) return ok;
    if (rt_layer_decode_workspace_bytes(desc) > (size_t)RT_DECODE_STATIC_SCRATCH_BYTES)
        return rt::set_error(RT_ERR_WORKSPACE, "this shape needs more scratch than the static array holds "
                                               "(RT_DECODE_STATIC_SCRATCH_BYTES); use rt_layer_decode_step", "");
    void* ws = nullptr;
    const rt_status st = device_scratch(&ws);
    if (st != RT_OK) return st;
    return rt_layer_decode_step(desc, w, n_past, x_t, z_t, k_cache, v_cache, ws,
                                (size_t)RT_DECODE_STATIC_SCRATCH_BYTES, stream);
}
