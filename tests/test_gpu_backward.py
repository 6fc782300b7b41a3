"""GPU parity of the blocked-schedule attention backward (and the forward that
saves its log-sum-exp) against the CPU oracle, through the C ABI.

Inputs are seeded and synthetic; the output adjoint a_bar is N(0,1) fp32.
Bars on every gradient, relative L2 against the oracle's fp64 gradient:
fp32 inputs 1e-5 (fp32 arithmetic over sums of up to N terms); bf16 inputs
5e-3: the stored attention output a is bf16 (as the forward keeps it), and
delta = <a_bar, a> enters every score's gradient, so a's half-ulp rounding
(2^-9 relative) reaches the gradients at that level; the MFMA rectangles
(blocks of 32 pairs and more) also round a_bar, the probabilities and the
score gradients to bf16 as product operands, each again 2^-9 relative.
"""
import math

import numpy as np
import pytest

import blocked_prefill_amd as rt
import oracle
import rt_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

BAR = {"f32": 1e-5, "bf16": 5e-3}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()


def _case(seed, n, b, h, dh, dt):
    w = rt_inputs.Workload("attn_case", b, n, h * dh, h, dh, 0, 0, dt, seed, update_only=True)
    t = rt_inputs.attn_inputs(w)
    t["a_bar"] = np.random.default_rng(seed + 1).standard_normal((n, b, h, dh)).astype(np.float32)
    return t


def _run(t, dt, scale, fill=None):
    import torch
    q, ke, ve, k, v = (G.dev(t[n], dt) for n in ("q", "k_eph", "v_eph", "k", "v"))
    N, B, H, dh = q.shape
    desc = G.attn_desc(B, N, H, dh, dt, scale)
    f32 = dict(dtype=torch.float32, device="cuda")
    a = torch.empty_like(q)
    lse = torch.empty((N, B, H), **f32)
    m, l = torch.empty((N, B, H), **f32), torch.empty((N, B, H), **f32)
    o = torch.empty((N, B, H, dh), **f32)
    rt.rt_attn_forward(desc, q, ke, ve, k, v, a, lse, m, l, o)
    ab = G.dev(t["a_bar"], "f32")
    outs = {n: torch.empty((N, B, H, dh), **f32) for n in ("q", "k_eph", "v_eph", "k", "v")}
    if fill is not None:
        for x in outs.values():
            x.fill_(fill)
    delta = torch.empty((N, B, H), **f32)
    rt.rt_attn_backward(desc, q, ke, ve, k, v, a, lse, ab, outs["q"], outs["k_eph"], outs["v_eph"], outs["k"],
                        outs["v"], delta)
    torch.cuda.synchronize()
    return a, lse, outs


def _check(got, want, dt, what):
    err = got - want
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(want), 1e-300))
    assert np.all(np.isfinite(got)), what
    assert rel <= BAR[dt], f"{what}: rel-L2 {rel:.3g} (max-abs {np.abs(err).max():.3g}) over {BAR[dt]}"
    print(f"{what}: rel-L2 {rel:.3g}")
    return rel


def test_forward_saves_the_log_sum_exp():
    """lse of every query against the scores written out in numpy (fp64, base 2)."""
    n, b, h, dh, scale = 70, 2, 2, 64, 0.125
    t = _case(21, n, b, h, dh, "bf16")
    a, lse, _ = _run(t, "bf16", scale)
    G.parity(G.host(a), oracle.attention(*(t[k] for k in ("q", "k_eph", "v_eph", "k", "v")), scale), "bf16", "a")
    q, k, ke = (t[x].astype(np.float64) for x in ("q", "k", "k_eph"))
    s2 = scale * math.log2(math.e)
    want = np.empty((n, b, h))
    for j in range(n):
        sc = np.concatenate([np.einsum("bhd,ibhd->ibh", q[j], k[:j]), np.einsum("bhd,bhd->bh", q[j], ke[j])[None]]) * s2
        mx = sc.max(0)
        want[j] = mx + np.log2(np.exp2(sc - mx).sum(0))
    assert np.abs(G.host(lse) - want).max() < 1e-4


@pytest.mark.parametrize("dt,n,b,h,dh", [
    ("bf16", 300, 3, 8, 64), ("bf16", 1000, 1, 1, 64), ("bf16", 70, 2, 4, 32), ("f32", 77, 2, 3, 32),
    ("bf16", 3, 2, 2, 64), ("bf16", 2, 2, 2, 64), ("bf16", 1, 2, 2, 64),
])
def test_forward_by_levels_equals_the_step_sequence(dt, n, b, h, dh):
    """rt_attn_forward runs each level of the schedule in one launch (largest
    blocks first); its outputs equal the steps t = 1..N-1 run one launch each
    (rt_update_finalize_step, as a layer runs them) bit for bit: every query
    merges the same blocks in the same order. P = 24 takes the two-pairs-per-wave
    kernel at 16 pairs, P = 1 the SIMT kernel there."""
    import torch
    t = _case(41 + n, n, b, h, dh, dt)
    scale = 1.0 / math.sqrt(dh)
    a_levels, _, _ = _run(t, dt, scale)
    desc = G.attn_desc(b, n, h, dh, dt, scale)
    q, ke, ve, k, v = (G.dev(t[x], dt) for x in ("q", "k_eph", "v_eph", "k", "v"))
    f32 = dict(dtype=torch.float32, device="cuda")
    m, l, o = torch.empty((n, b, h), **f32), torch.empty((n, b, h), **f32), torch.empty((n, b, h, dh), **f32)
    a_steps = torch.full_like(q, float("nan"))
    rt.rt_finalize_step(desc, 1, q, ke, ve, m, l, o, a_steps[0])
    for s_ in range(1, n):  # step s_ fused with the finish of position s_+1, one launch each
        rt.rt_update_finalize_step(desc, s_, q, ke, ve, k, v, m, l, o, a_steps[s_])
    torch.cuda.synchronize()
    assert torch.equal(a_levels, a_steps)


@pytest.mark.parametrize("dt,n,b,h,dh", [
    ("f32", 77, 2, 3, 32), ("f32", 1, 2, 2, 64), ("f32", 65, 1, 2, 128),
    ("bf16", 300, 3, 8, 64), ("bf16", 129, 2, 4, 128), ("bf16", 200, 3, 2, 32),
])
def test_attention_backward_matches_oracle(dt, n, b, h, dh):
    t = _case(31 + n, n, b, h, dh, dt)
    scale = 1.0 / math.sqrt(dh)
    _, _, outs = _run(t, dt, scale, fill=float("nan"))  # every output element is written
    ref = oracle.attention_backward(*(t[k] for k in ("q", "k_eph", "v_eph", "k", "v", "a_bar")), scale)
    for name in ("q", "k_eph", "v_eph", "k", "v"):
        _check(G.host(outs[name]), ref[name], dt, f"{name}_bar[{dt},{n},{b},{h},{dh}]")


def test_attention_backward_full_size_sampled_rows():
    """The isolated-update workload (B=64, 8 heads x 64, N=4096, bf16): every block
    size up to 2048; batch rows are independent, so sampled rows are exact."""
    w = rt_inputs.WORKLOADS["update_b64_n4096"]
    t = rt_inputs.attn_inputs(w)
    t["a_bar"] = np.random.default_rng(4096).standard_normal(t["q"].shape).astype(np.float32)
    scale = 1.0 / math.sqrt(w.head_dim)
    _, _, outs = _run(t, "bf16", scale)
    rows = [0, 37]
    ref = oracle.attention_backward(*(t[k][:, rows] for k in ("q", "k_eph", "v_eph", "k", "v", "a_bar")), scale)
    for name in ("q", "k_eph", "v_eph", "k", "v"):
        _check(G.host(outs[name])[:, rows], ref[name], "bf16", f"{name}_bar (full size)")
