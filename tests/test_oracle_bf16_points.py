"""Pins of the oracle's bf16 mode, one rounding point at a time.

The GPU library holds some tensors of the Recurrent Transformer layer in bf16
between its kernels; the oracle's bf16 mode (rt_oracle.c, round_bf16) rounds
exactly those to the nearest bf16 (ties to even) and computes everything else
in fp64. Which tensors are rounded, and where the rounded value (rather than
the exact one) is read, is the oracle's reading of the layer's storage
formats; the GPU parity tests rest on it, so each rounding point is pinned
here on its own.

Every stage of the layer (reading note lshu.cn/news/403416, translated paper
sections 2-2.2) is recomputed in torch fp64 from the oracle's own reported
values before their rounding (q, k', v', a, h, g, z, k, v), rounding exactly
where the reading says:
  q, k', v'  = W_{q,k,v} RMS_attn(x)            x is given in bf16
  a_t        = Attn over bf16(k_j), bf16(v_j) (j < t) and bf16(k'_t), bf16(v'_t),
               query bf16(q_t)
  h          = x + rho W_o bf16(a)
  g          = GELU(W_1 (g_mlp * bf16(h)) / rms(h))   rms of the exact h
  z          = h + rho W_2 bf16(g)                     residual: the exact h
  k, v       = W_{k,v} RMS_attn(bf16(z))               the stored output
  x_next     = bf16(z)
Each recomputation must equal the oracle's value to 1e-12, and the same
recomputation with that one rounding point dropped (the exact value read
instead) must miss it by far more, so a dropped or moved rounding point in
the oracle fails the matching test.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

torch.set_default_dtype(torch.float64)

N, R, D, H, FF = 12, 2, 64, 2, 128
DH = D // H
SIGMA, RHO, EPS = 0.3, 0.8, 1e-6
NAMES = ("z", "k", "v", "q", "k_eph", "v_eph", "a", "h", "g")


def _bf(a):
    """Nearest bf16 (ties to even), the rounding pinned against torch's cast in test_oracle_pins."""
    return oracle.round_bf16(np.asarray(a, dtype=np.float64))


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.fixture(scope="module")
def case():
    rng = np.random.default_rng(91)
    x = _bf(rng.standard_normal((N, R, D))).astype(np.float32)
    w = {
        "w_q": rng.standard_normal((D, D)) / math.sqrt(D), "w_k": rng.standard_normal((D, D)) / math.sqrt(D),
        "w_v": rng.standard_normal((D, D)) / math.sqrt(D), "w_o": rng.standard_normal((D, D)) / math.sqrt(D),
        "w_1": rng.standard_normal((FF, D)) / math.sqrt(D), "w_2": rng.standard_normal((D, FF)) / math.sqrt(FF),
    }
    w = {k: _bf(v).astype(np.float32) for k, v in w.items()}
    w["g_attn"] = (1 + 0.25 * rng.standard_normal(D)).astype(np.float32)
    w["g_mlp"] = (1 + 0.25 * rng.standard_normal(D)).astype(np.float32)
    out = oracle.layer_forward(x, w, n_heads=H, softmax_scale=SIGMA, residual_scale=RHO, rms_eps=EPS,
                               round_bf16=True, want=NAMES)
    W = {k: _t(v) for k, v in w.items()}
    return x, W, out


def _attention(q, ke, ve, k, v):
    """Position t's query over the persistent pairs j < t and its own ephemeral pair, per head."""
    q, ke, ve, k, v = (_t(a).reshape(N, R, H, DH).permute(1, 2, 0, 3) for a in (q, ke, ve, k, v))  # [R][H][N][dh]
    s_p = SIGMA * q @ k.transpose(-1, -2)                                     # [R][H][N][N]
    s_p = s_p.masked_fill(~torch.ones(N, N, dtype=torch.bool).tril(-1), float("-inf"))
    s_e = SIGMA * (q * ke).sum(-1, keepdim=True)                              # [R][H][N][1]
    p = torch.softmax(torch.cat([s_p, s_e], -1), -1)
    a = p[..., :N] @ v + p[..., N:] * ve
    return a.permute(2, 0, 1, 3).reshape(N, R, D).numpy()


def _pin(got, with_rounding, without_rounding, what):
    assert _rel(with_rounding, got) <= 1e-12, f"{what}: the stated rounding point does not reproduce the oracle"
    assert _rel(without_rounding, got) >= 1e-5, f"{what}: the test cannot tell the rounding point is there"


def test_projections_of_the_input_read_x_as_given(case):
    x, W, out = case
    u = F.rms_norm(_t(x), (D,), weight=W["g_attn"], eps=EPS)
    for name, wn in (("q", "w_q"), ("k_eph", "w_k"), ("v_eph", "w_v")):
        assert _rel(F.linear(u, W[wn]).numpy(), out[name]) <= 1e-12, name


def test_attention_reads_bf16_queries_pairs_and_cache(case):
    _, _, o = case
    got = o["a"]
    exact = _attention(o["q"], o["k_eph"], o["v_eph"], o["k"], o["v"])
    stored = _attention(_bf(o["q"]), _bf(o["k_eph"]), _bf(o["v_eph"]), _bf(o["k"]), _bf(o["v"]))
    assert _rel(stored, got) <= 1e-12
    assert _rel(exact, got) >= 1e-5
    # each operand on its own: reading that one exactly breaks the match
    for i, name in enumerate(("q", "k_eph", "v_eph", "k", "v")):
        args = [_bf(o[n]) for n in ("q", "k_eph", "v_eph", "k", "v")]
        args[i] = o[name]
        assert _rel(_attention(*args), got) >= 1e-6, f"{name} is read rounded"


def test_output_projection_reads_bf16_attention(case):
    x, W, o = case
    X = _t(x)
    _pin(o["h"], (X + RHO * F.linear(_t(_bf(o["a"])), W["w_o"])).numpy(),
         (X + RHO * F.linear(_t(o["a"]), W["w_o"])).numpy(), "h")


def test_mlp_up_reads_bf16_h_with_the_rms_of_the_exact_h(case):
    _, W, o = case
    h = _t(o["h"])
    rms = torch.sqrt((h * h).mean(-1, keepdim=True) + EPS)
    hb = _t(_bf(o["h"]))
    gelu = lambda u: F.gelu(u)  # exact erf form
    got = o["g"]
    want = gelu(F.linear(hb * W["g_mlp"], W["w_1"]) / rms).numpy()
    _pin(got, want, gelu(F.linear(h * W["g_mlp"], W["w_1"]) / rms).numpy(), "g (operand)")
    rms_b = torch.sqrt((hb * hb).mean(-1, keepdim=True) + EPS)
    assert _rel(gelu(F.linear(hb * W["g_mlp"], W["w_1"]) / rms_b).numpy(), got) >= 1e-7, "rms is of the exact h"


def test_mlp_down_reads_bf16_g_and_the_exact_h(case):
    _, W, o = case
    h = _t(o["h"])
    _pin(o["z"], (h + RHO * F.linear(_t(_bf(o["g"])), W["w_2"])).numpy(),
         (h + RHO * F.linear(_t(o["g"]), W["w_2"])).numpy(), "z")
    assert _rel((_t(_bf(o["h"])) + RHO * F.linear(_t(_bf(o["g"])), W["w_2"])).numpy(), o["z"]) >= 1e-5


def test_persistent_pair_reads_the_stored_output(case):
    _, W, o = case
    us = F.rms_norm(_t(_bf(o["z"])), (D,), weight=W["g_attn"], eps=EPS)
    ue = F.rms_norm(_t(o["z"]), (D,), weight=W["g_attn"], eps=EPS)
    for name, wn in (("k", "w_k"), ("v", "w_v")):
        _pin(o[name], F.linear(us, W[wn]).numpy(), F.linear(ue, W[wn]).numpy(), name)


def test_next_layer_input_is_the_rounded_output(case):
    _, _, o = case
    assert np.array_equal(o["x_next"].astype(np.float64), _bf(o["z"]))
    assert not np.array_equal(o["x_next"].astype(np.float64), o["z"])
