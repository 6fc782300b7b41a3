"""GPU parity of the layer's variants against the CPU oracle, through the C ABI:
the naive schedule, the standard Transformer layer (pairs from the input,
causal attention over all positions at once) and the decode step against a
persistent KV cache.

The oracle computes every variant position by position (naive schedule); the
Transformer layer is its kv_from_input mode. Inputs are seeded and synthetic.
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


def _weights(seed, d, f, dt):
    rng = np.random.default_rng(seed)
    w = {
        "w_q": rng.standard_normal((d, d)) / math.sqrt(d), "w_k": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_v": rng.standard_normal((d, d)) / math.sqrt(d), "w_o": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_1": rng.standard_normal((f, d)) / math.sqrt(d), "w_2": rng.standard_normal((d, f)) / math.sqrt(f),
    }
    return {k: rt_inputs.to_storage(v.astype(np.float32), dt) for k, v in w.items()}


def _input(seed, n, b, d, dt):
    return rt_inputs.to_storage(np.random.default_rng(seed).standard_normal((n, b, d)).astype(np.float32), dt)


def _forward(desc, x, w, dt):
    import torch
    buf = G.LayerBuffers(desc, G.dev(x, dt), w, dt, gains="g_attn" in w)
    buf.forward()
    torch.cuda.synchronize()
    return buf


# ---------------------------------------------------------------- naive schedule

@pytest.mark.parametrize("dt,n,b,d,h,f", [("bf16", 100, 3, 256, 4, 512), ("f32", 45, 2, 96, 3, 128),
                                           ("bf16", 70, 2, 256, 8, 256), ("bf16", 256, 16, 384, 6, 768)])
def test_naive_schedule_layer_matches_oracle(dt, n, b, d, h, f):
    """Query t+1 reads pairs 1..t in one pass (position counts below and above
    the MFMA kernel's 32, ragged tails); same result as the blocked schedule.
    At N*B = 4096 rows with d = 384 the up-front projection is a tall product
    whose 384-column segments are not whole 256-column tiles. bf16 results are
    held to the bar with the oracle's own noise floor over the recurrence
    (oracle_with_floor), as every bf16 layer test of tens of positions or more."""
    x = _input(n, n, b, d, dt)
    w = _weights(n + 1, d, f, dt)
    scale = 1.0 / math.sqrt(d // h)
    naive = _forward(G.layer_desc(b, n, d, h, f, dt, scale, flags=rt.RT_FLAG_NAIVE_SCHEDULE), x, w, dt)
    blocked = _forward(G.layer_desc(b, n, d, h, f, dt, scale), x, w, dt)
    if dt == "bf16":
        ref, floor = G.oracle_with_floor(x, w, n_heads=h, softmax_scale=scale)
    else:
        ref, floor = oracle.layer_forward(x, w, n_heads=h, softmax_scale=scale), {}
    for name in ("z", "k", "v"):
        m = G.parity(G.host(getattr(naive, name)), ref[name], dt, f"naive.{name}", floor=floor.get(name))
        G.parity(G.host(getattr(blocked, name)), ref[name], dt, f"blocked.{name}", floor=floor.get(name))
        print(f"naive {dt} N={n} B={b} d={d}: {name} {m}")


# ---------------------------------------------------------------- standard Transformer layer

@pytest.mark.parametrize("dt,n,b,d,h,f", [
    ("bf16", 300, 2, 256, 4, 512),   # MFMA causal attention: 3 query tiles of 128, ragged last tile
    ("bf16", 512, 8, 256, 4, 512),   # N*B = 4096 rows: the tall-GEMM tiles
    ("bf16", 256, 16, 384, 6, 768),  # 384-column outputs (q|k|v segments, W_o, W_2): 128-wide tall tiles
    ("bf16", 77, 3, 256, 8, 384),    # head_dim 32: SIMT causal attention
    ("f32", 60, 2, 96, 3, 128),
])
def test_transformer_layer_matches_oracle(dt, n, b, d, h, f):
    x = _input(2 * n + b, n, b, d, dt)
    w = _weights(n + 7, d, f, dt)
    scale = 1.0 / math.sqrt(d // h)
    buf = _forward(G.layer_desc(b, n, d, h, f, dt, scale, flags=rt.RT_FLAG_TRANSFORMER), x, w, dt)
    ref = oracle.layer_forward(x, w, n_heads=h, softmax_scale=scale, round_bf16=(dt == "bf16"),
                               kv_from_input=True)
    for name in ("z", "k", "v"):
        G.parity(G.host(getattr(buf, name)), ref[name], dt, f"transformer.{name}")


def test_transformer_layer_plan_replays_match_eager():
    import torch
    n, b, d, h, f = 200, 3, 256, 4, 512
    x = _input(9, n, b, d, "bf16")
    w = _weights(10, d, f, "bf16")
    buf = _forward(G.layer_desc(b, n, d, h, f, "bf16", 0.125, flags=rt.RT_FLAG_TRANSFORMER), x, w, "bf16")
    z0 = buf.z.clone()
    plan = buf.plan()
    for _ in range(2):
        buf.z.fill_(float("nan"))
        torch.cuda.synchronize()
        plan.launch()
        torch.cuda.synchronize()
        assert torch.equal(buf.z, z0)
    plan.destroy()


# ---------------------------------------------------------------- decode against the cache

def _qk_gains(w, seed, d):
    rng = np.random.default_rng(seed)
    w = dict(w)
    w["g_q"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    w["g_k"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    return w


@pytest.mark.parametrize("dt,n,b,d,h,f,flags", [
    ("bf16", 100, 3, 256, 4, 512, 0),                          # head_dim 64, blocked schedule
    ("bf16", 70, 2, 256, 8, 256, 0),                           # head_dim 32
    ("f32", 45, 2, 96, 3, 128, 0),
    ("bf16", 300, 2, 256, 4, 512, 4),                          # Transformer layer (RT_FLAG_TRANSFORMER)
    ("bf16", 40, 2, 256, 4, 512, 2),                           # naive schedule
])
def test_qk_norm_layer_matches_oracle(dt, n, b, d, h, f, flags):
    """Per-head query/key norm with non-unit gains (and non-unit RMS gains g_attn,
    g_mlp), on every layer mode."""
    x = _input(3 * n, n, b, d, dt)
    w = _qk_gains(_weights(n + 11, d, f, dt), n, d)
    rng = np.random.default_rng(n + 12)
    w["g_attn"] = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    w["g_mlp"] = (1 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    scale = 1.0 / math.sqrt(d // h)
    buf = _forward(G.layer_desc(b, n, d, h, f, dt, scale, flags=flags | rt.RT_FLAG_QK_NORM), x, w, dt)
    kw = dict(n_heads=h, softmax_scale=scale, qk_norm=True, kv_from_input=bool(flags & rt.RT_FLAG_TRANSFORMER))
    ref, floor = G.oracle_with_floor(x, w, **kw) if dt == "bf16" else (oracle.layer_forward(x, w, **kw), {})
    for name in ("z", "k", "v"):
        m = G.parity(G.host(getattr(buf, name)), ref[name], dt, f"qk_norm[{flags}].{name}", floor=floor.get(name))
        print(f"qk_norm[{flags}] {dt} N={n}: {name} {m}")


def _decode_case(dt, n_past, steps, b, d, h, f, flags=0, seed=0, scale=None):
    """Prefill positions 1..n_past with rt_layer_forward into caches of capacity
    n_past+steps, then decode positions n_past+1..n_past+steps one by one.
    Returns (z of the decoded positions, caches) as host arrays and the oracle's
    outputs over all n_past+steps positions."""
    import torch
    n = n_past + steps
    x = _input(seed + n, n, b, d, dt)
    w = _weights(seed + n + 1, d, f, dt)
    if flags & rt.RT_FLAG_QK_NORM:
        w = _qk_gains(w, seed + n + 2, d)
    scale = 1.0 / math.sqrt(d // h) if scale is None else scale
    td = G.torch_dtype(dt)
    kc = torch.full((n, b, d), float("nan"), dtype=td, device="cuda")
    vc = torch.full((n, b, d), float("nan"), dtype=td, device="cuda")
    x_dev = G.dev(x, dt)
    W = {k: G.dev(v, "f32" if k.startswith("g_") else dt) for k, v in w.items()}  # gains are fp32
    if n_past:
        pre = G.layer_desc(b, n_past, d, h, f, dt, scale, flags=flags)
        z_pre = torch.empty((n_past, b, d), dtype=td, device="cuda")
        ws = torch.empty(rt.rt_layer_workspace_bytes(pre), dtype=torch.uint8, device="cuda")
        # the caches are position-major: their first n_past rows are the prefill's caches
        rt.rt_layer_forward(pre, W, x_dev[:n_past], z_pre, kc[:n_past], vc[:n_past], ws)
    desc = G.layer_desc(b, n, d, h, f, dt, scale, flags=flags)
    ws = torch.empty(rt.rt_layer_decode_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    z = torch.empty((steps, b, d), dtype=td, device="cuda")
    for i in range(steps):
        rt.rt_layer_decode_step(desc, W, n_past + i, x_dev[n_past + i], z[i], kc, vc, ws)
    torch.cuda.synchronize()
    kw = dict(n_heads=h, softmax_scale=scale, kv_from_input=bool(flags & rt.RT_FLAG_TRANSFORMER),
              qk_norm=bool(flags & rt.RT_FLAG_QK_NORM))
    if dt == "bf16":
        ref, floor = G.oracle_with_floor(x, w, **kw)
    else:
        ref, floor = oracle.layer_forward(x, w, **kw), {}
    ref["floor"] = floor
    return G.host(z), G.host(kc), G.host(vc), ref


@pytest.mark.parametrize("dt,n_past,h,scale", [
    ("bf16", 0, 4, None), ("bf16", 1, 4, None), ("bf16", 14, 4, None), ("bf16", 31, 4, None), ("bf16", 32, 4, None),
    ("bf16", 45, 4, None), ("bf16", 129, 4, None), ("bf16", 100, 8, None), ("f32", 37, 4, None),
    ("bf16", 45, 4, 0.0),
])
def test_decode_steps_match_oracle(dt, n_past, h, scale):
    """Decode after a prefill of n_past positions (none, fewer than 32, ragged
    multiples of the 64-position tile), three positions in a row; softmax_scale
    0 (uniform weights) also across the masked rows of a ragged tile. n_past = 14:
    the third step reads 16 cached pairs, the two-pairs-per-wave kernel with no
    stored state (a null-state step of 8 or 16 pairs once faulted there)."""
    steps, b, d, f = 3, 3, 256, 512
    z, kc, vc, ref = _decode_case(dt, n_past, steps, b, d, h, f, scale=scale)
    n = n_past + steps
    fl = ref["floor"]
    G.parity(z, ref["z"][n_past:], dt, f"decode.z (n_past={n_past})", floor=fl.get("z"))
    G.parity(kc, ref["k"], dt, f"decode.k_cache (n_past={n_past})", floor=fl.get("k"))
    G.parity(vc, ref["v"], dt, f"decode.v_cache (n_past={n_past})", floor=fl.get("v"))
    assert kc.shape[0] == n


def test_qk_norm_decode_steps_match_oracle():
    steps, b, d, h, f, n_past = 3, 2, 256, 4, 512, 45
    z, kc, vc, ref = _decode_case("bf16", n_past, steps, b, d, h, f, flags=rt.RT_FLAG_QK_NORM, seed=9)
    fl = ref["floor"]
    G.parity(z, ref["z"][n_past:], "bf16", "qk_norm decode.z", floor=fl["z"])
    G.parity(kc, ref["k"], "bf16", "qk_norm decode.k_cache", floor=fl["k"])
    G.parity(vc, ref["v"], "bf16", "qk_norm decode.v_cache", floor=fl["v"])


@pytest.mark.parametrize("n_past", [0, 50])
def test_transformer_decode_steps_match_oracle(n_past):
    steps, b, d, h, f = 2, 2, 256, 4, 512
    z, kc, vc, ref = _decode_case("bf16", n_past, steps, b, d, h, f, flags=rt.RT_FLAG_TRANSFORMER, seed=5)
    G.parity(z, ref["z"][n_past:], "bf16", f"transformer decode.z (n_past={n_past})")
    G.parity(kc, ref["k"], "bf16", "transformer decode.k_cache")
    G.parity(vc, ref["v"], "bf16", "transformer decode.v_cache")


def test_zero_softmax_scale_is_uniform_attention():
    """softmax_scale = 0 gives every pair the same weight: the attention output of
    position 46 is the mean of values 1..45 and its ephemeral value (closed form)."""
    import torch
    b, h, dh, n_past = 2, 2, 64, 45
    n = n_past + 1
    t = rt_inputs.attn_inputs(rt_inputs.Workload("decode_case", b, n, h * dh, h, dh, 0, 0, "bf16", 77,
                                                 update_only=True))
    q, ke, ve, k, v = (G.dev(t[k_], "bf16") for k_ in ("q", "k_eph", "v_eph", "k", "v"))
    desc = G.attn_desc(b, n, h, dh, "bf16", 0.0)
    m = torch.empty((n, b, h), dtype=torch.float32, device="cuda")
    l, o = torch.empty_like(m), torch.empty((n, b, h, dh), dtype=torch.float32, device="cuda")
    a = torch.empty((b, h * dh), dtype=torch.bfloat16, device="cuda")
    # the blocked path of the same position, then the mean over the pairs
    for t_ in range(1, n):
        rt.rt_blocked_attn_update(desc, t_, q, k, v, m, l, o)
    rt.rt_finalize_step(desc, n, q, ke, ve, m, l, o, a)
    torch.cuda.synchronize()
    want = (t["v"][:n_past].astype(np.float64).sum(0) + t["v_eph"][n_past]) / n
    G.parity(G.host(a).reshape(b, h, dh), want, "bf16", "uniform attention")


def test_decode_full_size_after_prefill():
    """B=512, d=1024, 16 heads x 64: decode position 2049 after the 2048-position
    prefill (the persistent cache of the bench's layer), two sampled rows."""
    import torch
    wl = rt_inputs.WORKLOADS["stack6_d1024_b512_n2048"]
    n_past = wl.n_pos
    scale = 1.0 / math.sqrt(wl.head_dim)
    w = rt_inputs.layer_weights(wl, 0)
    x = rt_inputs.layer_input(wl)
    x_new = rt_inputs.to_storage(np.random.default_rng(2049).standard_normal((wl.batch, wl.d_model))
                                 .astype(np.float32), "bf16")
    td = torch.bfloat16
    kc = torch.empty((n_past + 1, wl.batch, wl.d_model), dtype=td, device="cuda")
    vc = torch.empty_like(kc)
    W = {k: G.dev(v, "bf16") for k, v in w.items() if k.startswith("w_")}
    pre = G.layer_desc(wl.batch, n_past, wl.d_model, wl.n_heads, wl.d_ff, "bf16", scale)
    z_pre = torch.empty((n_past, wl.batch, wl.d_model), dtype=td, device="cuda")
    ws = torch.empty(rt.rt_layer_workspace_bytes(pre), dtype=torch.uint8, device="cuda")
    rt.rt_layer_forward(pre, W, G.dev(x, "bf16"), z_pre, kc[:n_past], vc[:n_past], ws)
    del ws, z_pre
    desc = G.layer_desc(wl.batch, n_past + 1, wl.d_model, wl.n_heads, wl.d_ff, "bf16", scale)
    ws = torch.empty(rt.rt_layer_decode_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    z = torch.empty((wl.batch, wl.d_model), dtype=td, device="cuda")
    rt.rt_layer_decode_step(desc, W, n_past, G.dev(x_new, "bf16"), z, kc, vc, ws)
    torch.cuda.synchronize()
    rows = [0, 511]
    xr = np.concatenate([x[:, rows], x_new[None, rows]], axis=0)
    ref = oracle.layer_forward(xr, w, n_heads=wl.n_heads, softmax_scale=scale, round_bf16=True)
    G.parity(G.host(z)[rows], ref["z"][n_past], "bf16", "decode (full size).z")
    G.parity(G.host(kc[n_past])[rows], ref["k"][n_past], "bf16", "decode (full size).k")
    G.parity(G.host(vc[n_past])[rows], ref["v"][n_past], "bf16", "decode (full size).v")
