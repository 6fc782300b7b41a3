"""GPU tests of the layer stack (rt_stack_forward, rt_stack_plan_create).

Blocked layers run as a wavefront with chunked query projections and deferred
rows of large blocks; every query still merges the same blocks in the same
order as when the layers run one after another. Checked here:
- fp32: the stack equals the layers run one after another, bit for bit (the
  fp32 products and updates compute each output element alone, so launch
  grouping and row ranges cannot change a value);
- bf16: every layer of the stack meets the parity bars against the oracle on
  that layer's actual input (the stack's own previous output), and against
  the library's single-layer path on the same input;
- the plan replays the eager stack bit for bit; the naive schedule, the
  Transformer layer and one-layer stacks equal the single-layer path.
Inputs are seeded and synthetic.
"""
import math

import numpy as np
import pytest

import blocked_prefill_amd as rt
import oracle
import rt_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()


def _weights(seed, d, f, dt, gains=True, qk=False):
    rng = np.random.default_rng(seed)
    w = {
        "w_q": rng.standard_normal((d, d)) / math.sqrt(d), "w_k": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_v": rng.standard_normal((d, d)) / math.sqrt(d), "w_o": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_1": rng.standard_normal((f, d)) / math.sqrt(d), "w_2": rng.standard_normal((d, f)) / math.sqrt(f),
    }
    w = {k: rt_inputs.to_storage(v.astype(np.float32), dt) for k, v in w.items()}
    if gains:
        w["g_attn"] = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32)
        w["g_mlp"] = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    if qk:
        w["g_q"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
        w["g_k"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    return w


def _dev_weights(w, dt):
    return {k: G.dev(v, "f32" if k.startswith("g_") else dt) for k, v in w.items()}


class StackBuffers:
    """Device buffers of a stack forward."""

    def __init__(self, desc, x_dev, weights, dt):
        import torch
        N, B, D = desc.attn.seq_len, desc.attn.batch, desc.d_model
        self.desc, self.x, self.dt = desc, x_dev, dt
        self.w = [_dev_weights(w, dt) for w in weights]
        td = G.torch_dtype(dt)
        L = len(weights)
        self.z = [torch.full((N, B, D), float("nan"), dtype=td, device="cuda") for _ in range(L)]
        self.k = [torch.full((N, B, D), float("nan"), dtype=td, device="cuda") for _ in range(L)]
        self.v = [torch.full((N, B, D), float("nan"), dtype=td, device="cuda") for _ in range(L)]
        nbytes = rt.rt_stack_workspace_bytes(desc, L)
        assert nbytes == L * rt.rt_layer_workspace_bytes(desc), rt.rt_last_error()
        self.ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-filled scratch

    def forward(self):
        rt.rt_stack_forward(self.desc, self.w, self.x, self.z, self.k, self.v, self.ws)

    def plan(self):
        return rt.rt_stack_plan_create(self.desc, self.w, self.x, self.z, self.k, self.v, self.ws)


def _layer(desc, x_dev, w, dt):
    """One layer through the single-layer entry point (device outputs)."""
    import torch
    buf = G.LayerBuffers(desc, x_dev, w, dt, gains="g_attn" in w)
    buf.forward()
    torch.cuda.synchronize()
    return buf


def _case(dt, n, b, d, h, f, n_layers, seed, gains=True, qk=False, flags=0, rho=1.0):
    x = rt_inputs.to_storage(np.random.default_rng(seed).standard_normal((n, b, d)).astype(np.float32), dt)
    ws = [_weights(seed + 1 + i, d, f, dt, gains=gains, qk=qk) for i in range(n_layers)]
    scale = 1.0 / math.sqrt(d // h)
    desc = G.layer_desc(b, n, d, h, f, dt, scale, rho=rho, flags=flags)
    return x, ws, scale, desc


def _run_stack(desc, x, ws, dt):
    import torch
    st = StackBuffers(desc, G.dev(x, dt), ws, dt)
    st.forward()
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("n", [300, 37, 2, 1])
def test_stack_f32_equals_layer_by_layer(n):
    """N=300: chunks of 16 positions, so steps of 32..256 pairs defer rows; N=37:
    chunks of 8, the step of 16 pairs defers rows 25..32; N=1 and 2: each layer's
    whole sequence inside the lag."""
    import torch
    dt, b, d, h, f, L = "f32", 2, 96, 3, 128, 3
    x, ws, scale, desc = _case(dt, n, b, d, h, f, L, seed=10 + n)
    st = _run_stack(desc, x, ws, dt)
    xin = st.x
    for i in range(L):
        one = _layer(desc, xin, ws[i], dt)
        for name in ("z", "k", "v"):
            got, want = getattr(st, name)[i], getattr(one, name)
            assert torch.equal(got, want), f"layer {i}.{name}: max diff {float((got - want).abs().max())}"
        xin = one.z


@pytest.mark.parametrize("n,qk,rho,gains,h", [(100, False, 1.0, True, 4), (100, False, 1.0 / math.sqrt(6.0), True, 4),
                                             (100, True, 1.0, True, 4), (100, False, 1.0, True, 8),
                                             (300, False, 1.0, True, 4), (300, True, 1.0, True, 4)])
def test_stack_bf16_each_layer_matches_oracle(n, qk, rho, gains, h):
    """Every layer of a bf16 stack, with data flowing from the oracle to the GPU only:
    - the oracle runs its own chain (layer l reads its own stored output of layer l-1);
    - the library's single-layer path on the oracle's input of layer l meets the bars
      against the oracle's layer l;
    - the stack's layer l meets the bars against the single-layer path on the stack's
      own input of layer l (the wavefront's grouped products and deferred rows against
      one layer's launches);
    - the stack's layer 0 (same input as the oracle's) meets the bars against it.
    N=100 has chunks of 8 positions (steps of 16..64 pairs defer rows); N=300 chunks
    of 16 (steps of 32..256). h = 8: head_dim 32, whose small steps run per layer."""
    dt, b, d, f, L = "bf16", 3, 256, 512, 3
    flags = rt.RT_FLAG_QK_NORM if qk else 0
    x, ws, scale, desc = _case(dt, n, b, d, h, f, L, seed=20 + n, qk=qk, flags=flags, rho=rho, gains=gains)
    st = _run_stack(desc, x, ws, dt)
    x_oracle = x
    for i in range(L):
        ref, floor = G.oracle_with_floor(x_oracle, ws[i], n_heads=h, softmax_scale=scale, residual_scale=rho,
                                         qk_norm=qk)
        on_oracle_input = _layer(desc, G.dev(x_oracle, dt), ws[i], dt)
        on_stack_input = _layer(desc, st.x if i == 0 else st.z[i - 1], ws[i], dt)
        for name in ("z", "k", "v"):
            m = G.parity(G.host(getattr(on_oracle_input, name)), ref[name], dt, f"layer {i}.{name} vs oracle",
                         floor=floor[name])
            # two bf16 results of the same layer (the oracle's floor of this layer stands for the
            # noise between two rounding orders)
            s_ = G.parity(G.host(getattr(st, name)[i]), G.host(getattr(on_stack_input, name)), dt,
                          f"stack layer {i}.{name} vs single layer", floor=floor[name], stored=True)
            if i == 0:
                G.parity(G.host(getattr(st, name)[0]), ref[name], dt, f"stack layer 0.{name} vs oracle",
                         floor=floor[name])
            print(f"layer {i}.{name}: single layer vs oracle {m}; stack vs single layer {s_}")
        x_oracle = ref["x_next"]


def test_stack_plan_replays_match_eager():
    import torch
    dt = "bf16"
    x, ws, scale, desc = _case(dt, 160, 3, 256, 4, 512, 2, seed=5)
    st = _run_stack(desc, x, ws, dt)
    ref = [t.clone() for t in st.z + st.k + st.v]
    plan = st.plan()
    for _ in range(3):
        for t in st.z + st.k + st.v:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        plan.launch()
        torch.cuda.synchronize()
        for got, want in zip(st.z + st.k + st.v, ref):
            assert torch.equal(got, want)
    plan.destroy()


@pytest.mark.parametrize("flags,n_layers", [(rt.RT_FLAG_NAIVE_SCHEDULE, 2), (rt.RT_FLAG_TRANSFORMER, 2), (0, 1)])
def test_stack_other_modes_equal_layer_by_layer(flags, n_layers):
    """Stacks that run layer after layer (the naive schedule, the Transformer
    layer, a single layer): bit for bit the single-layer path."""
    import torch
    dt = "bf16"
    x, ws, scale, desc = _case(dt, 70, 2, 256, 4, 512, n_layers, seed=7 + flags, flags=flags)
    st = _run_stack(desc, x, ws, dt)
    xin = st.x
    for i in range(n_layers):
        one = _layer(desc, xin, ws[i], dt)
        for name in ("z", "k", "v"):
            assert torch.equal(getattr(st, name)[i], getattr(one, name)), f"layer {i}.{name}"
        xin = one.z


def test_stack_full_d1024_b512_n2048_six_layers():
    """The 6-layer stack at full size (B=512, N=2048, d=1024, bf16) through the
    stack plan, as the benchmark runs it. Layer 0 reads the same input as the
    oracle: its sampled batch rows against the oracle. Every layer against the
    single-layer plan on the stack's own input of that layer (sampled rows; the
    single-layer path on the oracle's own chain is checked against the oracle
    layer by layer in test_gpu_parity)."""
    import torch
    wl = rt_inputs.WORKLOADS["stack6_d1024_b512_n2048"]
    rows = [0, 1, 255, 511]
    scale = 1.0 / math.sqrt(wl.head_dim)
    desc = G.layer_desc(wl.batch, wl.n_pos, wl.d_model, wl.n_heads, wl.d_ff, "bf16", scale)
    x = rt_inputs.layer_input(wl)
    weights = [rt_inputs.layer_weights(wl, i) for i in range(wl.n_layers)]
    weights = [{k: w[k] for k in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")} for w in weights]
    st = StackBuffers(desc, G.dev(x, "bf16"), weights, "bf16")
    del x
    plan = st.plan()
    plan.launch()
    torch.cuda.synchronize()
    plan.destroy()
    del st.ws
    idx = torch.tensor(rows, device="cuda")
    x_rows = rt_inputs.layer_input(wl, rows=rows[:2]).astype(np.float64)
    ref, floor = G.oracle_with_floor(x_rows, weights[0], n_heads=wl.n_heads, softmax_scale=scale)
    m = {nm: G.parity(G.host(getattr(st, nm)[0][:, idx[:2]]), ref[nm], "bf16", f"stack layer 0.{nm} vs oracle",
                      floor=floor[nm]) for nm in ("z", "k", "v")}
    print(f"stack layer 0 vs oracle: {m}", flush=True)
    for i in range(wl.n_layers):
        buf = G.LayerBuffers(desc, st.x if i == 0 else st.z[i - 1], weights[i], "bf16")
        p = buf.plan()
        p.launch()
        torch.cuda.synchronize()
        p.destroy()
        m = {nm: G.parity(G.host(getattr(st, nm)[i][:, idx]), G.host(getattr(buf, nm)[:, idx]), "bf16",
                          f"stack layer {i}.{nm} vs single layer", floor=floor[nm], stored=True)
             for nm in ("z", "k", "v")}
        print(f"stack layer {i} vs the single-layer plan on its input: {m}", flush=True)
        del buf
