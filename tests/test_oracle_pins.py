"""Pins of the CPU oracle against facts that do not come from the oracle itself.

The oracle (oracle/rt_oracle.c) runs the naive schedule of the Recurrent
Transformer layer (reading note lshu.cn/news/403416, translated paper sections
2-2.2, summary sections 2.2 and 4.1). Each test below would fail on a plausible
mistake in it:
  * bf16 rounding   -- against torch's fp32->bf16 cast and hand-worked ties;
  * RMSNorm / GELU  -- against torch.nn.functional in fp64;
  * attention       -- reduces to torch's causal scaled_dot_product_attention
                       when the persistent pairs equal the ephemeral ones;
                       a_1 = v'_1 exactly; uniform weights at softmax scale 0;
                       equals the blocked algorithm (exactness claim, summary
                       section 4.2) to 1e-12 in fp64;
  * the layer       -- with the persistent pair taken from the input it is the
                       textbook pre-LN Transformer layer (section 2.1: the RT
                       layer differs only in where the exposed pair comes
                       from), written here with torch.nn.functional; with W_q=0
                       position 2 attends uniformly to a pair built from the
                       output z_1 (section 2.2); blocked == naive; batch rows
                       are independent.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import blocked_reference as blocked

torch.set_default_dtype(torch.float64)


def _rng(seed):
    return np.random.default_rng(seed)


def _weights(rng, d, f, scale=1.0):
    w = {
        "w_q": rng.standard_normal((d, d)) / math.sqrt(d) * scale,
        "w_k": rng.standard_normal((d, d)) / math.sqrt(d) * scale,
        "w_v": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_o": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_1": rng.standard_normal((f, d)) / math.sqrt(d),
        "w_2": rng.standard_normal((d, f)) / math.sqrt(f),
        "g_attn": 1.0 + 0.25 * rng.standard_normal(d),
        "g_mlp": 1.0 + 0.25 * rng.standard_normal(d),
    }
    return {k: v.astype(np.float32) for k, v in w.items()}


def _rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


# ---------------------------------------------------------------- bf16 rounding

def test_round_bf16_matches_torch_cast_on_fp32_values():
    rng = _rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
        rng.standard_normal(2000).astype(np.float32) * np.float32(1e-39),  # fp32 subnormals
        np.array([0.0, -0.0, 3.3895313892515355e38, -3.4e38]),
    ]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, want)


def test_round_bf16_ties_go_to_even():
    e = 2.0 ** -8
    cases = {1 + e: 1.0, 1 + 3 * e: 1 + 4 * e, -(1 + e): -1.0, 2 + 2 * e: 2.0, 2 + 6 * e: 2 + 8 * e,
             1 + e * (1 + 2 ** -20): 1 + 2 * e}
    for x, want in cases.items():
        assert oracle.round_bf16(np.array([x]))[0] == want, x


# ---------------------------------------------------------------- sub-operations

def test_rmsnorm_matches_torch():
    rng = _rng(2)
    for n in (1, 7, 64, 1024):
        x = rng.standard_normal(n) * 3.0
        g = (1.0 + rng.standard_normal(n)).astype(np.float32)
        want = F.rms_norm(torch.from_numpy(x), (n,), weight=torch.from_numpy(g.astype(np.float64)), eps=1e-6)
        assert np.allclose(oracle.rmsnorm(x, g, 1e-6), want.numpy(), rtol=1e-13, atol=1e-14)


def test_gelu_matches_torch_exact_erf():
    u = np.linspace(-9, 9, 4001)
    want = F.gelu(torch.from_numpy(u), approximate="none").numpy()
    assert np.allclose(oracle.gelu(u), want, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- attention

def _attn_tensors(rng, n, r, h, dh):
    return [rng.standard_normal((n, r, h, dh)).astype(np.float32) for _ in range(5)]


@pytest.mark.parametrize("n,r,h,dh", [(1, 1, 1, 4), (17, 2, 3, 8), (64, 3, 2, 32)])
def test_attention_reduces_to_causal_sdpa(n, r, h, dh):
    rng = _rng(3)
    q, k, v = (rng.standard_normal((n, r, h, dh)).astype(np.float32) for _ in range(3))
    sigma = 1.0 / math.sqrt(dh)
    got = oracle.attention(q, k, v, k, v, sigma)  # persistent pairs equal the ephemeral ones
    tq, tk, tv = (torch.from_numpy(a.astype(np.float64)).permute(1, 2, 0, 3) for a in (q, k, v))
    want = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=sigma).permute(2, 0, 1, 3).numpy()
    assert _rel(got, want) < 1e-13


def test_attention_first_position_is_its_ephemeral_value():
    rng = _rng(4)
    q, ke, ve, k, v = _attn_tensors(rng, 5, 3, 2, 16)
    a = oracle.attention(q, ke, ve, k, v, 0.37)
    assert np.array_equal(a[0], ve[0].astype(np.float64))


def test_attention_zero_scale_is_uniform_average():
    rng = _rng(5)
    q, ke, ve, k, v = _attn_tensors(rng, 9, 2, 2, 8)
    a = oracle.attention(q, ke, ve, k, v, 0.0)
    for t in range(9):
        want = (v[:t].astype(np.float64).sum(axis=0) + ve[t]) / (t + 1)
        assert np.allclose(a[t], want, rtol=1e-13, atol=1e-14)


def test_attention_ignores_pairs_at_or_after_own_position():
    rng = _rng(6)
    q, ke, ve, k, v = _attn_tensors(rng, 12, 2, 2, 8)
    a = oracle.attention(q, ke, ve, k, v, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[7:] = 100.0
    v2[7:] = -50.0
    a2 = oracle.attention(q, ke, ve, k2, v2, 0.5)
    assert np.array_equal(a[:8], a2[:8])       # position t reads persistent pairs 1..t-1 only
    assert not np.allclose(a[8:], a2[8:])


def test_attention_at_selected_positions_equals_full():
    rng = _rng(7)
    t = _attn_tensors(rng, 40, 3, 2, 16)
    full = oracle.attention(*t, 0.3)
    sel = [40, 1, 17, 2, 33]
    part = oracle.attention_at(*t, 0.3, sel)
    assert np.array_equal(part, full[np.array(sel) - 1])


@pytest.mark.parametrize("n", [1, 2, 3, 8, 37, 64])
def test_attention_blocked_equals_naive(n):
    rng = _rng(10 + n)
    t = _attn_tensors(rng, n, 2, 2, 16)
    a_naive = oracle.attention(*t, 0.25)
    a_blk = blocked.attention(*t, 0.25)
    assert _rel(a_blk, a_naive) <= 1e-12


# ---------------------------------------------------------------- the layer

def _textbook_transformer_layer(x, w, n_heads, sigma, rho, eps, qk_norm=False):
    """Pre-LN causal Transformer layer (section 2.1 of the translated paper) in torch fp64.
    qk_norm: torch's RMS norm over each head's query and key, times gains g_q, g_k."""
    X = torch.from_numpy(x.astype(np.float64))                       # [N][R][d]
    W = {k: torch.from_numpy(v.astype(np.float64)) for k, v in w.items()}
    n, r, d = X.shape
    dh = d // n_heads
    u = F.rms_norm(X, (d,), weight=W["g_attn"], eps=eps)
    split = lambda y: y.reshape(n, r, n_heads, dh)
    norm = (lambda y, g: F.rms_norm(y, (dh,), eps=eps) * g.reshape(n_heads, dh)) if qk_norm else (lambda y, g: y)
    heads = lambda y: y.permute(1, 2, 0, 3)                            # [R][H][N][dh]
    kq = norm(split(F.linear(u, W["w_k"])), W.get("g_k"))
    q = heads(norm(split(F.linear(u, W["w_q"])), W.get("g_q")))
    k, v = heads(kq), heads(split(F.linear(u, W["w_v"])))
    a = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=sigma).permute(2, 0, 1, 3).reshape(n, r, d)
    h = X + rho * F.linear(a, W["w_o"])
    y = h + rho * F.linear(F.gelu(F.linear(F.rms_norm(h, (d,), weight=W["g_mlp"], eps=eps), W["w_1"])), W["w_2"])
    us = F.rms_norm(X, (d,), weight=W["g_attn"], eps=eps)
    return {"z": y.numpy(), "k": kq.reshape(n, r, d).numpy(), "v": F.linear(us, W["w_v"]).numpy(),
            "a": a.numpy(), "h": h.numpy()}


@pytest.mark.parametrize("n,r,d,h,f,rho", [(1, 1, 16, 2, 32, 1.0), (23, 2, 32, 4, 64, 1.0), (40, 3, 64, 2, 256, 0.5)])
def test_layer_with_input_kv_is_the_textbook_transformer(n, r, d, h, f, rho):
    rng = _rng(20 + n)
    x = rng.standard_normal((n, r, d)).astype(np.float32)
    w = _weights(rng, d, f)
    sigma = 1.0 / math.sqrt(d // h)
    got = oracle.layer_forward(x, w, n_heads=h, softmax_scale=sigma, residual_scale=rho, rms_eps=1e-6,
                               kv_from_input=True, want=("z", "k", "v", "a", "h"))
    want = _textbook_transformer_layer(x, w, h, sigma, rho, 1e-6)
    for name in ("z", "k", "v", "a", "h"):
        assert _rel(got[name], want[name]) < 1e-12, name


@pytest.mark.parametrize("n,r,d,h,f", [(1, 1, 16, 2, 32), (23, 2, 32, 4, 64), (30, 2, 64, 2, 128)])
def test_qk_norm_layer_with_input_kv_is_the_textbook_transformer(n, r, d, h, f):
    """The query/key norm (translated paper section 2 notation, per head) against
    torch's RMS norm applied to each head of the textbook layer's q and k."""
    rng = _rng(60 + n)
    x = rng.standard_normal((n, r, d)).astype(np.float32)
    w = _weights(rng, d, f)
    w["g_q"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    w["g_k"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    sigma = 1.0 / math.sqrt(d // h)
    got = oracle.layer_forward(x, w, n_heads=h, softmax_scale=sigma, rms_eps=1e-6, kv_from_input=True,
                               qk_norm=True, want=("z", "k", "v", "a", "h"))
    want = _textbook_transformer_layer(x, w, h, sigma, 1.0, 1e-6, qk_norm=True)
    for name in ("z", "k", "v", "a", "h"):
        assert _rel(got[name], want[name]) < 1e-12, name
    if n > 1:  # (one position attends to its own pair only: no score matters)
        plain = oracle.layer_forward(x, w, n_heads=h, softmax_scale=sigma, rms_eps=1e-6, kv_from_input=True)
        assert _rel(plain["z"], want["z"]) > 1e-3  # the norm changes the layer


def test_qk_norm_makes_the_layer_invariant_to_query_and_key_scale():
    """With the per-head query/key norm, scaling W_q and W_k by positive constants
    leaves the RT layer unchanged (up to the norm's epsilon); without it, not."""
    rng = _rng(70)
    n, r, d, h, f = 12, 2, 32, 4, 64
    x = rng.standard_normal((n, r, d)).astype(np.float32)
    w = _weights(rng, d, f)
    w2 = dict(w, w_q=(w["w_q"] * 8).astype(np.float32), w_k=(w["w_k"] * 0.25).astype(np.float32))
    kw = dict(n_heads=h, softmax_scale=0.3, rms_eps=1e-30)
    a, b = oracle.layer_forward(x, w, qk_norm=True, **kw), oracle.layer_forward(x, w2, qk_norm=True, **kw)
    for name in ("z", "k", "v"):
        assert _rel(a[name], b[name]) < 1e-12, name
    c, e = oracle.layer_forward(x, w, **kw), oracle.layer_forward(x, w2, **kw)
    assert _rel(c["z"], e["z"]) > 1e-3


def test_persistent_pair_comes_from_the_output():
    """W_q = 0 makes every score 0: position 2's output is then the uniform average
    of the value built from z_1 (the first position's layer output) and its own
    ephemeral value; z_1 itself is the textbook Transformer layer's first output."""
    rng = _rng(30)
    d, h, f = 32, 4, 64
    x = rng.standard_normal((2, 1, d)).astype(np.float32)
    w = _weights(rng, d, f)
    w["w_q"] = np.zeros_like(w["w_q"])
    eps = 1e-6
    got = oracle.layer_forward(x, w, n_heads=h, softmax_scale=0.125, rms_eps=eps, want=("z", "a", "v"))
    first = _textbook_transformer_layer(x[:1], w, h, 0.125, 1.0, eps)
    assert _rel(got["z"][0], first["z"][0]) < 1e-13
    Wt = {k: torch.from_numpy(v.astype(np.float64)) for k, v in w.items()}
    z1 = torch.from_numpy(first["z"][0, 0])
    v1 = F.linear(F.rms_norm(z1, (d,), weight=Wt["g_attn"], eps=eps), Wt["w_v"])
    v2e = F.linear(F.rms_norm(torch.from_numpy(x[1, 0].astype(np.float64)), (d,), weight=Wt["g_attn"], eps=eps),
                   Wt["w_v"])
    assert _rel(got["a"][1, 0], ((v1 + v2e) / 2).numpy()) < 1e-13
    assert _rel(got["v"][0, 0], v1.numpy()) < 1e-13
    # and it is not what the Transformer layer (pair from x_1) would give
    v1x = F.linear(F.rms_norm(torch.from_numpy(x[0, 0].astype(np.float64)), (d,), weight=Wt["g_attn"], eps=eps),
                   Wt["w_v"])
    assert _rel(got["a"][1, 0], ((v1x + v2e) / 2).numpy()) > 1e-3


@pytest.mark.parametrize("n,kv_in,qk", [(1, False, False), (2, False, False), (3, False, False), (8, False, False),
                                        (37, False, False), (37, True, False), (64, False, False), (37, False, True),
                                        (20, True, True)])
def test_layer_blocked_equals_naive(n, kv_in, qk):
    rng = _rng(40 + n)
    d, h, f, r = 32, 2, 64, 2
    x = rng.standard_normal((n, r, d)).astype(np.float32)
    w = _weights(rng, d, f)
    if qk:
        w["g_q"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
        w["g_k"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    got = oracle.layer_forward(x, w, n_heads=h, softmax_scale=0.3, residual_scale=0.8, kv_from_input=kv_in,
                               qk_norm=qk)
    want = blocked.layer_forward(x, w, n_heads=h, softmax_scale=0.3, residual_scale=0.8, kv_from_input=kv_in,
                                 qk_norm=qk)
    for name in ("z", "k", "v"):
        assert _rel(got[name], want[name]) <= 1e-12, name


def test_batch_rows_are_independent():
    rng = _rng(50)
    n, r, d, h, f = 20, 5, 32, 2, 64
    x = rng.standard_normal((n, r, d)).astype(np.float32)
    w = _weights(rng, d, f)
    perm = np.array([3, 0, 4, 1, 2])
    a = oracle.layer_forward(x, w, n_heads=h, softmax_scale=0.2)
    b = oracle.layer_forward(x[:, perm], w, n_heads=h, softmax_scale=0.2)
    for name in ("z", "k", "v"):
        assert np.array_equal(a[name][:, perm], b[name])


def test_bf16_emulation_stores_bf16_values_and_stays_close():
    rng = _rng(60)
    n, r, d, h, f = 30, 2, 64, 2, 128
    x = oracle.round_bf16(rng.standard_normal((n, r, d))).astype(np.float32)
    w = {k: oracle.round_bf16(v.astype(np.float64)).astype(np.float32) for k, v in _weights(rng, d, f).items()}
    emu = oracle.layer_forward(x, w, n_heads=h, softmax_scale=0.125, round_bf16=True)
    ref = oracle.layer_forward(x, w, n_heads=h, softmax_scale=0.125, round_bf16=False)
    xs = emu["x_next"].astype(np.float64)
    assert np.array_equal(xs, oracle.round_bf16(emu["z"]))
    assert _rel(emu["z"], ref["z"]) < 2e-2
    assert _rel(emu["z"], ref["z"]) > 0.0


@pytest.mark.parametrize("n,qk", [(1, False), (8, False), (37, False), (20, True)])
def test_literal_kv_source_blocked_equals_naive(n, qk):
    """The literal reading of the cut persistent-pair formula (translated paper
    section 2.2): k_t = W_k z_t, v_t = W_v z_t without the RMS; the blocked
    schedule reaches the naive result there too."""
    rng = _rng(80 + n)
    d, h, f, r = 32, 2, 64, 2
    x = rng.standard_normal((n, r, d)).astype(np.float32)
    w = _weights(rng, d, f)
    if qk:
        w["g_q"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
        w["g_k"] = (1 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    kw = dict(n_heads=h, softmax_scale=0.3, residual_scale=0.8, qk_norm=qk, kv_source_norm=False)
    got = oracle.layer_forward(x, w, **kw)
    want = blocked.layer_forward(x, w, **kw)
    for name in ("z", "k", "v"):
        assert _rel(got[name], want[name]) <= 1e-12, name
    if n > 1:
        normed = oracle.layer_forward(x, w, **dict(kw, kv_source_norm=True))
        assert _rel(got["z"], normed["z"]) > 1e-3  # the two readings differ


def test_literal_kv_source_reads_the_output_itself():
    """W_q = 0 (uniform weights): position 2's output is the mean of W_v z_1, the
    value built from the first position's output with no RMS, and of its own
    ephemeral value W_v RMS_attn(x_2)."""
    rng = _rng(31)
    d, h, f = 32, 4, 64
    x = rng.standard_normal((2, 1, d)).astype(np.float32)
    w = _weights(rng, d, f)
    w["w_q"] = np.zeros_like(w["w_q"])
    eps = 1e-6
    got = oracle.layer_forward(x, w, n_heads=h, softmax_scale=0.125, rms_eps=eps, kv_source_norm=False,
                               want=("z", "a", "v", "k"))
    Wt = {k: torch.from_numpy(v.astype(np.float64)) for k, v in w.items()}
    z1 = torch.from_numpy(got["z"][0, 0])
    v1 = F.linear(z1, Wt["w_v"])
    v2e = F.linear(F.rms_norm(torch.from_numpy(x[1, 0].astype(np.float64)), (d,), weight=Wt["g_attn"], eps=eps),
                   Wt["w_v"])
    assert _rel(got["v"][0, 0], v1.numpy()) < 1e-13
    assert _rel(got["k"][0, 0], F.linear(z1, Wt["w_k"]).numpy()) < 1e-13
    assert _rel(got["a"][1, 0], ((v1 + v2e) / 2).numpy()) < 1e-13
    # z_1 does not depend on the reading (position 1 sees only its own pair)
    first = _textbook_transformer_layer(x[:1], w, h, 0.125, 1.0, eps)
    assert _rel(got["z"][0], first["z"][0]) < 1e-13


def test_round_bf16_vector_and_c_forms_agree():
    """The oracle's vectorised rounding and its C form (used inside the layer) agree."""
    rng = _rng(2)
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-45, 40, 3000),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.3961e38, 1e-45, 2.0 ** -134, 2.0 ** -133 * 1.5])])
    got = oracle.round_bf16(v)
    want = np.array([oracle.round_bf16_scalar(x) for x in v])
    assert np.array_equal(got, want)
