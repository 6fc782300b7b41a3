// Host-side checks of the C ABI for a sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only): every call below returns
// from argument validation or from pure host logic before any HIP call, so
// the program needs no GPU. It exits non-zero on a wrong status; the
// sanitizers abort on a memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "../../include/rt_prefill.h"

static int failures = 0;

static void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, rt_last_error());
        ++failures;
    }
}

int main() {
    void* const fake = reinterpret_cast<void*>(uintptr_t(1) << 20);  // aligned, never dereferenced
    rt_attn_desc a{};
    a.batch = 2; a.seq_len = 16; a.n_heads = 2; a.head_dim = 64; a.dtype = RT_BF16; a.softmax_scale = 0.125f;
    rt_layer_desc d{};
    d.attn = a; d.d_model = 128; d.d_ff = 256; d.rms_eps = 1e-6f; d.residual_scale = 1.f; d.kv_source_norm = 1;
    rt_layer_weights w{};
    w.w_q = w.w_k = w.w_v = w.w_o = w.w_1 = w.w_2 = fake;

    // the schedule rule, every step of a few lengths
    for (int32_t n : {1, 7, 64, 100, 32768}) {
        for (int32_t t = 1; t <= n; t += (n > 1000 ? 97 : 1)) {
            int32_t k0, k1, q0, q1;
            expect(rt_schedule_step(t, n, &k0, &k1, &q0, &q1) == RT_OK, "schedule step");
            const int32_t b = t & -t;
            expect(k0 == t - b + 1 && k1 == t && q0 == t + 1 && q1 == (t + b < n ? t + b : n), "schedule values");
        }
    }
    int32_t k0, k1, q0, q1;
    expect(rt_schedule_step(0, 4, &k0, &k1, &q0, &q1) == RT_ERR_INVALID_ARG, "schedule t = 0");
    expect(rt_schedule_step(1, 4, nullptr, &k1, &q0, &q1) == RT_ERR_INVALID_ARG, "schedule null output");

    // workspace sizes and descriptor validation
    const size_t ws = rt_layer_workspace_bytes(&d);
    expect(ws > 0, "workspace bytes");
    expect(rt_stack_workspace_bytes(&d, 6) == 6 * ws, "stack workspace bytes");
    expect(rt_layer_decode_workspace_bytes(&d) > 0, "decode workspace bytes");
    expect(rt_layer_backward_workspace_bytes(&d) > ws, "backward workspace bytes");
    rt_layer_desc bad = d;
    bad.d_model = 100;
    expect(rt_layer_workspace_bytes(&bad) == 0, "bad d_model");
    bad = d;
    bad.kv_source_norm = 3;
    expect(rt_layer_workspace_bytes(&bad) == 0, "bad kv_source_norm");
    bad = d;
    bad.flags = 64;
    expect(rt_layer_forward(&bad, &w, fake, fake, fake, fake, fake, ws, nullptr) == RT_ERR_INVALID_ARG, "bad flags");
    expect(rt_layer_workspace_bytes(nullptr) == 0, "null descriptor");

    // pointer and size checks of every entry point
    expect(rt_layer_forward(&d, &w, fake, fake, fake, fake, fake, ws - 1, nullptr) == RT_ERR_WORKSPACE,
           "small workspace");
    expect(rt_layer_forward(&d, &w, nullptr, fake, fake, fake, fake, ws, nullptr) == RT_ERR_INVALID_ARG, "null x");
    expect(std::strstr(rt_last_error(), "x is NULL") != nullptr, "error text");
    rt_plan* plan = nullptr;
    expect(rt_layer_plan_create(&d, &w, fake, fake, fake, nullptr, fake, ws, &plan) == RT_ERR_INVALID_ARG,
           "plan null cache");
    expect(plan == nullptr, "no plan on failure");
    expect(rt_blocked_attn_update(&a, 0, fake, fake, fake, (float*)fake, (float*)fake, (float*)fake, nullptr) ==
               RT_ERR_INVALID_ARG,
           "update t = 0");
    expect(rt_blocked_attn_update(&a, 16, fake, fake, fake, (float*)fake, (float*)fake, (float*)fake, nullptr) ==
               RT_OK,
           "update at t = N is a no-op");
    expect(rt_finalize_step(&a, 2, fake, fake, fake, nullptr, nullptr, nullptr, fake, nullptr) == RT_ERR_INVALID_ARG,
           "finalize without state");
    expect(rt_layer_decode_step(&d, &w, 16, fake, fake, fake, fake, fake, 1u << 30, nullptr) == RT_ERR_INVALID_ARG,
           "decode past the cache");
    void* zs[2] = {fake, fake};
    expect(rt_stack_forward(&d, 2, nullptr, fake, zs, zs, zs, fake, 2 * ws, nullptr) == RT_ERR_INVALID_ARG,
           "stack null weights");
    rt_layer_grads g{};
    expect(rt_layer_backward(&d, &w, fake, fake, (const float*)fake, (float*)fake, &g, fake, 1u << 30, nullptr) ==
               RT_ERR_INVALID_ARG,
           "backward null gradients");
    expect(std::strlen(rt_last_error()) < 512, "bounded error text");
    std::printf("abi_check: %d failures\n", failures);
    return failures ? 1 : 0;
}
