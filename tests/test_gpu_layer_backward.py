"""GPU parity of the RT layer's backward (rt_layer_backward) against the
oracle's gradient (oracle/layer_backward.py, fp64), through the C ABI.

The backward is evaluated at a forward pass; data flows from the oracle to
the GPU only: the GPU's rt_layer_backward reads the oracle's own stored
output z (its bf16 values in bf16 layers) as the forward it differentiates,
and the oracle takes its derivatives at its own forward values, in bf16
layers as a bf16 layer stores them (q, k', v', k, v, a, z, the MLP's
pre-activation and activation, the normalised inputs of the weight products;
round_bf16 of layer_backward).

Inputs are seeded and synthetic: x ~ N(0,1), weights N(0, 1/d_in), gains
1 + 0.3 N(0,1) where present, z_bar ~ N(0,1).

Bar, relative L2 of each gradient against the oracle's: 1e-5 in fp32
layers, 5e-3 in bf16 layers (the stated bf16 bar; what remains is the bf16
rounding of the adjoints where a product reads them, 2^-9 relative each,
and the rounding decisions of the recomputed forward values).
"""
import math

import numpy as np
import pytest

import blocked_prefill_amd as rt
import rt_inputs
from oracle.layer_backward import layer_backward
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BAR = {"f32": 1e-5, "bf16": 5e-3}
NAMES = ("x", "w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()


def _case(seed, n, b, d, f, gains):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, b, d)).astype(np.float32)
    w = {}
    for name, shape in (("w_q", (d, d)), ("w_k", (d, d)), ("w_v", (d, d)), ("w_o", (d, d)), ("w_1", (f, d)),
                        ("w_2", (d, f))):
        w[name] = (rng.standard_normal(shape) / math.sqrt(shape[1])).astype(np.float32)
    if gains:
        w["g_attn"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
        w["g_mlp"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    z_bar = rng.standard_normal((n, b, d)).astype(np.float32)
    return x, w, z_bar


def _run(dt, n, b, d, heads, f, rho, gains, seed):
    import torch
    x, w, z_bar = _case(seed, n, b, d, f, gains)
    if dt == "bf16":
        x = rt_inputs.to_storage(x, dt)
        w = {k: (rt_inputs.to_storage(v, dt) if k.startswith("w_") else v) for k, v in w.items()}
    scale = 1.0 / math.sqrt(d // heads)
    desc = G.layer_desc(b, n, d, heads, f, dt, scale, rho=rho)
    ref = layer_backward(x, w, z_bar.astype(np.float64), n_heads=heads, softmax_scale=scale, residual_scale=rho,
                         round_bf16=(dt == "bf16"))
    buf = G.LayerBuffers(desc, G.dev(x, dt), w, dt, gains=gains)
    if dt == "bf16":
        buf.z = G.dev(ref["z_stored"], dt)  # the forward being differentiated: the oracle's stored output
    else:
        buf.forward()
    f32 = dict(dtype=torch.float32, device="cuda")
    grads = {k: torch.full(w[k].shape, float("nan"), **f32) for k in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    grads["g_attn"] = torch.full((d,), float("nan"), **f32)
    grads["g_mlp"] = torch.full((d,), float("nan"), **f32)
    x_bar = torch.full((n, b, d), float("nan"), **f32)
    nbytes = rt.rt_layer_backward_workspace_bytes(desc)
    assert nbytes > 0, rt.rt_last_error()
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    zb = torch.from_numpy(z_bar).cuda()
    rt.rt_layer_backward(desc, buf.w, buf.x, buf.z, zb, x_bar, grads, ws)
    torch.cuda.synchronize()
    got = {"x": G.host(x_bar), **{k: G.host(v) for k, v in grads.items()}}
    return got, ref


@pytest.mark.parametrize("dt,n,b,d,heads,f,rho,gains", [
    ("f32", 20, 2, 64, 2, 128, 0.7, True),
    ("bf16", 100, 3, 256, 4, 512, 1.0, True),
    ("bf16", 64, 64, 256, 4, 512, 0.8, False),   # N*B = 4096 rows: the batched products' tall tiles
    # N*B = 16384 rows: the weight gradients in 16 K ranges of one launch, on 256x256 tiles where the
    # gradient has 256-column multiples (W_2's 384 x 768) and 128x128 where not (d = 384)
    ("bf16", 64, 256, 384, 6, 768, 0.9, False),
])
def test_layer_backward_matches_oracle(dt, n, b, d, heads, f, rho, gains):
    got, ref = _run(dt, n, b, d, heads, f, rho, gains, seed=500 + n)
    for name in NAMES:
        g, r = got[name], ref[name]
        assert np.all(np.isfinite(g)), f"{name}: non-finite (an element left unwritten?)"
        rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
        print(f"{dt} N={n} B={b} d={d}: {name} rel-L2 {rel:.3g}")
        assert rel <= BAR[dt], f"{name}: rel-L2 {rel:.3g} over {BAR[dt]}"


def test_layer_backward_full_size_two_rows():
    """The stack workload's layer shape (B=512, N=2048, d=1024, 16x64 heads,
    F=4096, bf16) with z_bar nonzero on two batch rows only. Batch rows are
    independent, so every adjoint of the other rows is exactly zero: x_bar
    vanishes there, and the weight gradients are those two rows' alone,
    which the oracle computes on the two rows."""
    import torch
    import rt_inputs
    n, b, d, heads, f = 2048, 512, 1024, 16, 4096
    rows = [3, 400]
    wl = rt_inputs.Workload("bwd_full", b, n, d, heads, d // heads, f, 1, "bf16", 77)
    x = rt_inputs.layer_input(wl)
    w = rt_inputs.layer_weights(wl, 0)
    w = {k: w[k] for k in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    z_bar = np.zeros((n, b, d), dtype=np.float32)
    z_bar[:, rows] = np.random.default_rng(78).standard_normal((n, len(rows), d)).astype(np.float32)
    scale = 1.0 / math.sqrt(d // heads)
    desc = G.layer_desc(b, n, d, heads, f, "bf16", scale)
    ref = layer_backward(x[:, rows], w, z_bar[:, rows].astype(np.float64), n_heads=heads, softmax_scale=scale,
                         round_bf16=True)
    buf = G.LayerBuffers(desc, G.dev(x, "bf16"), w, "bf16")
    buf.forward()  # the other rows' forward; the two rows take the oracle's stored output
    buf.z[:, torch.tensor(rows, device="cuda")] = G.dev(ref["z_stored"], "bf16")
    f32 = dict(dtype=torch.float32, device="cuda")
    grads = {k: torch.empty(w[k].shape, **f32) for k in w}
    x_bar = torch.empty((n, b, d), **f32)
    ws = torch.empty(rt.rt_layer_backward_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    zb = torch.from_numpy(z_bar).cuda()
    rt.rt_layer_backward(desc, buf.w, buf.x, buf.z, zb, x_bar, grads, ws)
    torch.cuda.synchronize()
    xb = G.host(x_bar)
    others = np.ones(b, dtype=bool)
    others[rows] = False
    assert np.all(xb[:, others] == 0.0)
    del ws, buf
    got = {"x": xb[:, rows], **{k: G.host(v) for k, v in grads.items()}}
    for name in ("x", "w_q", "w_k", "w_v", "w_o", "w_1", "w_2"):
        rel = float(np.linalg.norm(got[name] - ref[name]) / max(np.linalg.norm(ref[name]), 1e-300))
        print(f"full size, rows {rows}: {name} rel-L2 {rel:.3g}")
        assert rel <= BAR["bf16"], f"{name}: rel-L2 {rel:.3g} over {BAR['bf16']}"
