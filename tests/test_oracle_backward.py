"""Pins of the oracle's attention backward (the gradient of the RT attention map
for an output adjoint), each against something other than the oracle itself:

  - central finite differences of L = sum(a_bar * a) through the blocked
    numpy reference (fp64, a separate implementation of the forward);
  - torch's autograd of causal scaled-dot-product attention, to which the RT
    attention reduces when every persistent pair equals the ephemeral pair of
    the same position (then dk = k_bar + k'_bar, dv = v_bar + v'_bar);
  - the closed form at softmax_scale 0 (uniform weights).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import blocked_reference as blocked

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _case(seed, n, r, h, dh):
    rng = np.random.default_rng(seed)
    t = {name: rng.standard_normal((n, r, h, dh)).astype(np.float32) for name in ("q", "k_eph", "v_eph", "k", "v")}
    t["a_bar"] = rng.standard_normal((n, r, h, dh)).astype(np.float32)
    return t


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


@pytest.mark.parametrize("n,r,h,dh,sigma", [(1, 1, 1, 4, 0.5), (5, 2, 2, 4, 0.7), (9, 1, 3, 8, 0.35)])
def test_backward_matches_finite_differences(n, r, h, dh, sigma):
    t = _case(100 + n, n, r, h, dh)
    grads = oracle.attention_backward(*(t[k] for k in ("q", "k_eph", "v_eph", "k", "v", "a_bar")), sigma)
    abar = t["a_bar"].astype(np.float64)
    base = {k: t[k].astype(np.float64) for k in ("q", "k_eph", "v_eph", "k", "v")}

    def loss(args):
        return float(np.sum(abar * blocked.attention(*(args[k] for k in ("q", "k_eph", "v_eph", "k", "v")), sigma)))

    rng = np.random.default_rng(7)
    step = 1e-5
    for name in ("q", "k_eph", "v_eph", "k", "v"):
        flat = [tuple(int(rng.integers(0, s)) for s in base[name].shape) for _ in range(12)]
        for idx in flat:
            plus = {k: v.copy() for k, v in base.items()}
            minus = {k: v.copy() for k, v in base.items()}
            plus[name][idx] += step
            minus[name][idx] -= step
            fd = (loss(plus) - loss(minus)) / (2 * step)
            got = grads[name][idx]
            assert abs(got - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, got, fd)


@pytest.mark.parametrize("n,r,h,dh", [(1, 2, 1, 8), (17, 2, 2, 16), (40, 1, 3, 8)])
def test_backward_reduces_to_causal_sdpa_autograd(n, r, h, dh):
    t = _case(200 + n, n, r, h, dh)
    sigma = 1.0 / np.sqrt(dh)
    g = oracle.attention_backward(t["q"], t["k"], t["v"], t["k"], t["v"], t["a_bar"], sigma)
    to = lambda x: torch.tensor(x.astype(np.float64)).permute(1, 2, 0, 3).contiguous().requires_grad_(True)
    Q, K, V = to(t["q"]), to(t["k"]), to(t["v"])
    A = F.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=sigma)
    A.backward(torch.tensor(t["a_bar"].astype(np.float64)).permute(1, 2, 0, 3))
    back = lambda x: x.grad.permute(2, 0, 1, 3).numpy()
    assert _rel(g["q"], back(Q)) < 1e-12
    assert _rel(g["k"] + g["k_eph"], back(K)) < 1e-12
    assert _rel(g["v"] + g["v_eph"], back(V)) < 1e-12


def test_backward_at_zero_scale_is_the_uniform_average_closed_form():
    n, r, h, dh = 11, 2, 2, 4
    t = _case(300, n, r, h, dh)
    g = oracle.attention_backward(*(t[k] for k in ("q", "k_eph", "v_eph", "k", "v", "a_bar")), 0.0)
    ab = t["a_bar"].astype(np.float64)
    for name in ("q", "k_eph", "k"):
        assert np.all(g[name] == 0.0), name
    w = 1.0 / np.arange(1, n + 1)                                   # position t (0-based) averages t+1 pairs
    assert _rel(g["v_eph"], ab * w[:, None, None, None]) < 1e-14
    # persistent value i is read by every later position t > i with weight 1/(t+1)
    tail = np.cumsum((ab * w[:, None, None, None])[::-1], axis=0)[::-1]
    want = np.concatenate([tail[1:], np.zeros_like(tail[:1])])
    assert _rel(g["v"], want) < 1e-13
