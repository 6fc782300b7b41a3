"""Pins of the oracle's layer gradient (oracle/layer_backward.py), each against
something other than the oracle's own chain rule:

  - central differences of L = sum(z_bar * z) through rt_oracle.c's layer
    forward (IEEE double, no rounding), for sampled entries of the input,
    every weight matrix and both RMS gains;
  - torch's autograd (float64) of a separate torch implementation of the RT
    layer's forward written in this file (naive schedule, the same readings);
  - the closed form at residual_scale 0: z = x, so x_bar = z_bar and every
    weight and gain gradient is exactly zero.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.layer_backward import layer_backward

WEIGHTS = ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp")


def _case(seed, n, r, d, heads, f):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, r, d)).astype(np.float32)
    w = {}
    for name, shape in (("w_q", (d, d)), ("w_k", (d, d)), ("w_v", (d, d)), ("w_o", (d, d)), ("w_1", (f, d)),
                        ("w_2", (d, f))):
        w[name] = (rng.standard_normal(shape) / math.sqrt(shape[1])).astype(np.float32)
    w["g_attn"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    w["g_mlp"] = (1.0 + 0.3 * rng.standard_normal(d)).astype(np.float32)
    z_bar = rng.standard_normal((n, r, d))
    return x, w, z_bar


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300))


def test_layer_gradient_matches_central_differences():
    n, r, d, heads, f = 5, 2, 8, 2, 16
    sigma, rho = 1.0 / math.sqrt(d // heads), 0.8
    x, w, z_bar = _case(11, n, r, d, heads, f)
    g = layer_backward(x, w, z_bar, n_heads=heads, softmax_scale=sigma, residual_scale=rho)

    def loss(xx, ww):
        z = oracle.layer_forward(xx, ww, n_heads=heads, softmax_scale=sigma, residual_scale=rho, want=("z",))["z"]
        return float(np.sum(z_bar * z))

    rng = np.random.default_rng(5)
    for name in ("x",) + WEIGHTS:
        base = x if name == "x" else w[name]
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in base.shape)
            # the inputs are fp32: the actual steps are measured after rounding
            plus, minus = base.copy(), base.copy()
            plus[idx] = np.float32(base[idx] + np.float32(1e-3))
            minus[idx] = np.float32(base[idx] - np.float32(1e-3))
            hp = float(plus[idx]) - float(base[idx])
            hm = float(base[idx]) - float(minus[idx])
            args_p = (plus, w) if name == "x" else (x, {**w, name: plus})
            args_m = (minus, w) if name == "x" else (x, {**w, name: minus})
            fd = (loss(*args_p) - loss(*args_m)) / (hp + hm)
            got = g[name][idx]
            assert abs(got - fd) <= 2e-5 * max(1.0, abs(fd)), (name, idx, got, fd)


def _torch_layer(x, w, heads, sigma, rho, eps):
    """The RT layer's forward in torch (float64), naive schedule: a second implementation."""
    n, r, d = x.shape
    dh = d // heads

    def rms(t, g):
        return g * t / torch.sqrt((t * t).mean(-1, keepdim=True) + eps)

    keys, vals, zs = [], [], []
    for t in range(n):
        ux = rms(x[t], w["g_attn"])
        q, ke, ve = (ux @ w[m].T for m in ("w_q", "w_k", "w_v"))
        qh, keh, veh = (y.reshape(r, heads, dh) for y in (q, ke, ve))
        if keys:
            K = torch.stack(keys + [keh])            # [t+1][r][heads][dh], ephemeral pair last
            V = torch.stack(vals + [veh])
        else:
            K, V = keh[None], veh[None]
        s = sigma * torch.einsum("rhe,irhe->irh", qh, K)
        p = torch.softmax(s, dim=0)
        a = torch.einsum("irh,irhe->rhe", p, V).reshape(r, d)
        hh = x[t] + rho * a @ w["w_o"].T
        u = rms(hh, w["g_mlp"]) @ w["w_1"].T
        gact = 0.5 * u * (1.0 + torch.erf(u / math.sqrt(2.0)))
        z = hh + rho * gact @ w["w_2"].T
        zs.append(z)
        uz = rms(z, w["g_attn"])
        keys.append((uz @ w["w_k"].T).reshape(r, heads, dh))
        vals.append((uz @ w["w_v"].T).reshape(r, heads, dh))
    return torch.stack(zs)


@pytest.mark.parametrize("n,r,d,heads,f,rho", [(7, 2, 16, 2, 32, 1.0), (12, 1, 12, 3, 24, 0.5)])
def test_layer_gradient_matches_torch_autograd(n, r, d, heads, f, rho):
    sigma, eps = 1.0 / math.sqrt(d // heads), 1e-6
    x, w, z_bar = _case(20 + n, n, r, d, heads, f)
    g = layer_backward(x, w, z_bar, n_heads=heads, softmax_scale=sigma, residual_scale=rho, rms_eps=eps)
    xt = torch.tensor(x.astype(np.float64), requires_grad=True)
    wt = {k: torch.tensor(v.astype(np.float64), requires_grad=True) for k, v in w.items()}
    z = _torch_layer(xt, wt, heads, sigma, rho, eps)
    # the two forwards agree first
    zo = oracle.layer_forward(x, w, n_heads=heads, softmax_scale=sigma, residual_scale=rho, rms_eps=eps)["z"]
    assert _rel(z.detach().numpy(), zo) < 1e-12
    (z * torch.tensor(z_bar)).sum().backward()
    assert _rel(g["x"], xt.grad.numpy()) < 1e-10
    for name in WEIGHTS:
        assert _rel(g[name], wt[name].grad.numpy()) < 1e-10, name


def test_layer_gradient_at_zero_residual_scale_is_the_identity():
    n, r, d, heads, f = 6, 2, 8, 2, 16
    x, w, z_bar = _case(3, n, r, d, heads, f)
    g = layer_backward(x, w, z_bar, n_heads=heads, softmax_scale=0.5, residual_scale=0.0)
    assert np.array_equal(g["x"], z_bar)
    for name in WEIGHTS:
        assert np.all(g[name] == 0.0), name
