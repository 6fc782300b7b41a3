"""Helpers of the GPU parity tests: device tensors, the library's entry points
driven over whole sequences, and the parity bars.

Bars (fp32: relative L2 <= 1e-5; bf16: max |gpu - ref| <= 2e-2 and relative
L2 <= 5e-3) compare each tensor the GPU stores in bf16 with the oracle's value
of that tensor before its own rounding; the oracle rounds to bf16 where the
library holds bf16 between steps. A bf16 output cannot be closer to the exact
value than half its own unit in the last place (0.031 for |value| in [8, 16)),
so the bf16 max-abs bar applies to the error beyond that half-ulp; the raw
maximum is reported alongside.
"""
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import blocked_prefill_amd as rt  # noqa: E402

TOL = {"f32": {"rel_l2": 1e-5}, "bf16": {"rel_l2": 5e-3, "max_abs": 2e-2}}


def ensure_built():
    if not os.path.exists(rt.library_path):
        from blocked_prefill_amd import build
        build.build()
    rt.load()


def torch_dtype(dt):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


def rt_dtype(dt):
    return rt.RT_BF16 if dt == "bf16" else rt.RT_F32


def dev(a: np.ndarray, dt: str):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch_dtype(dt)).cuda()


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def parity(gpu, ref, dt: str, what: str = ""):
    """Return the metrics; raise AssertionError with them when the bar is missed."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = gpu - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(err))) if err.size else 0.0
    m = {"rel_l2": rel, "max_abs": mx}
    bar = TOL[dt]
    ok = rel <= bar["rel_l2"]
    if dt == "bf16" and err.size:
        excess = np.abs(err) - 0.5 * bf16_ulp(ref)
        i = int(np.argmax(excess))
        m["max_abs_beyond_half_ulp"] = float(excess.flat[i])
        m["at_ref"] = float(ref.flat[i])
        ok = ok and m["max_abs_beyond_half_ulp"] <= bar["max_abs"]
    assert ok, f"{what}: {m} over the bar {bar}"
    return m


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits; subnormal spacing 2^-133)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 2.0 ** -126)))
    return np.exp2(e - 7)


def attn_desc(batch, n_pos, n_heads, head_dim, dt, scale):
    return rt.AttnDesc(batch=batch, seq_len=n_pos, n_heads=n_heads, head_dim=head_dim, dtype=rt_dtype(dt),
                       softmax_scale=scale)


def layer_desc(batch, n_pos, d_model, n_heads, d_ff, dt, scale, eps=1e-6, rho=1.0, flags=0):
    a = attn_desc(batch, n_pos, n_heads, d_model // n_heads, dt, scale)
    return rt.LayerDesc(attn=a, d_model=d_model, d_ff=d_ff, rms_eps=eps, residual_scale=rho, flags=flags)


def run_attention_sequence(desc, q, ke, ve, k, v, state_fill=None):
    """Drive the blocked schedule through the C ABI: for t = 1..N, finalize(t)
    then update(t). Inputs are device tensors [N][B][H][dh]; returns a (device)."""
    import torch
    N, B, H, dh = q.shape
    m = torch.empty((N, B, H), dtype=torch.float32, device="cuda")
    l = torch.empty_like(m)
    o = torch.empty((N, B, H, dh), dtype=torch.float32, device="cuda")
    if state_fill is not None:
        for s in (m, l, o):
            s.fill_(state_fill)
    a = torch.empty((N, B, H * dh), dtype=q.dtype, device="cuda")
    for t in range(1, N + 1):
        rt.rt_finalize_step(desc, t, q, ke, ve, m, l, o, a[t - 1])
        rt.rt_blocked_attn_update(desc, t, q, k, v, m, l, o)
    torch.cuda.synchronize()
    return a.view(N, B, H, dh)


class LayerBuffers:
    """Device buffers of one layer forward."""

    def __init__(self, desc, x_dev, weights_np: dict, dt: str, gains: bool = False):
        import torch
        N, B = desc.attn.seq_len, desc.attn.batch
        D = desc.d_model
        self.desc = desc
        self.x = x_dev
        self.w = {n: dev(weights_np[n], dt) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
        if gains:
            for n in ("g_attn", "g_mlp"):
                self.w[n] = torch.from_numpy(np.ascontiguousarray(weights_np[n], dtype=np.float32)).cuda()
        for n in ("g_q", "g_k"):  # query/key norm gains (fp32), used with RT_FLAG_QK_NORM
            if weights_np.get(n) is not None:
                self.w[n] = torch.from_numpy(np.ascontiguousarray(weights_np[n], dtype=np.float32)).cuda()
        td = torch_dtype(dt)
        self.z = torch.empty((N, B, D), dtype=td, device="cuda")
        self.k = torch.empty((N, B, D), dtype=td, device="cuda")
        self.v = torch.empty((N, B, D), dtype=td, device="cuda")
        nbytes = rt.rt_layer_workspace_bytes(desc)
        assert nbytes > 0, rt.rt_last_error()
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def forward(self):
        rt.rt_layer_forward(self.desc, self.w, self.x, self.z, self.k, self.v, self.ws)

    def plan(self):
        return rt.rt_layer_plan_create(self.desc, self.w, self.x, self.z, self.k, self.v, self.ws)
