"""Gradient of the RT layer, in fp64 -- TEST INFRASTRUCTURE ONLY.

The layer (Recurrent Transformer reading note, lshu.cn/news/403416,
translated paper sections 2.1-2.2; the readings of rt_oracle.c): per position
t and batch row,
    u_x = RMS_attn(x_t);  q, k', v' = W_q u_x, W_k u_x, W_v u_x
    a_t = Attn over the persistent pairs 1..t-1 and the ephemeral pair (per head)
    h_t = x_t + rho W_o a_t;  m_t = RMS_mlp(h_t);  u_t = W_1 m_t
    z_t = h_t + rho W_2 GELU(u_t)
    u_z = RMS_attn(z_t);  k_t, v_t = W_k u_z, W_v u_z   (read by positions > t)
The pages give the backward only as a heading (translated paper section 6.4)
and the remark that it can be batched outside the position loop (section
6.1). What follows is the chain rule for L = sum(z_bar * z), written out:
  - positions are visited in reverse order. When position t is reached,
    every query > t has its adjoint, so the adjoints of k_t and v_t are
    complete; they reach z_t through RMS_attn:
        z_bar_t(total) = z_bar_t + RMS'(z_t)^T (W_k^T k_bar_t + W_v^T v_bar_t)
  - the MLP and the output projection are differentiated as usual:
        u_bar = rho (W_2^T z_bar_t) * GELU'(u_t)
        h_bar = z_bar_t + RMS'(h_t)^T (W_1^T u_bar);  a_bar = rho W_o^T h_bar
  - the attention of query t is differentiated as in rt_oracle.c's
    attention backward (softmax Jacobian, D = <a_bar, a>), adding into the
    adjoints of the earlier persistent pairs;
  - after the loop: x_bar = h_bar + RMS'(x)^T (W_q^T q_bar + W_k^T k'_bar +
    W_v^T v'_bar), and every weight gradient is a sum over positions and rows
    of an outer product (adjoint of a product's output times its input).
RMS(x) = g x / r with r = sqrt(mean(x^2) + eps) has the adjoint
    x_bar = g y_bar / r - x sum(g y_bar x) / (d r^3),  g_bar = sum(y_bar x / r).
With round_bf16 unset this is the gradient of the exact layer. With it set,
the derivatives are taken at the forward values a bf16 layer holds between
its kernels (rt_oracle.c's bf16 mode): q, k', v', the persistent k, v, the
attention output a and the output z as stored (rounded to bf16, RNE); the
MLP's pre-activation u = W_1 (g_mlp * bf16(h)) / rms(h) and its activation
GELU(u) as stored; and the normalised inputs of the weight products,
RMS_attn(x), RMS_attn(bf16(z)) and RMS_mlp(h), as stored. h stays exact
(a bf16 layer keeps it in fp32). The roundings themselves are taken as the
identity (they have no derivative), and the adjoints stay exact.
Plain numpy, loops over positions; the forward values come from rt_oracle.c.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf


def _rms_fwd(x, g, eps):
    """(RMS(x) with gain g, 1/r per row) over the last axis."""
    rinv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return g * x * rinv, rinv


def _rms_bwd(x, g, ybar, eps):
    """Adjoint of x for y = g x / r, and this call's contribution to g's adjoint."""
    d = x.shape[-1]
    rinv = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    gy = g * ybar
    xbar = gy * rinv - x * np.sum(gy * x, axis=-1, keepdims=True) * rinv ** 3 / d
    gbar = np.sum(ybar * x * rinv, axis=tuple(range(x.ndim - 1)))
    return xbar, gbar


def _gelu(u):
    return 0.5 * u * (1.0 + _erf(u / math.sqrt(2.0)))


def _gelu_grad(u):
    """d/du of u Phi(u): Phi(u) + u phi(u)."""
    return 0.5 * (1.0 + _erf(u / math.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def layer_backward(x, weights: dict, z_bar, *, n_heads: int, softmax_scale: float, residual_scale: float = 1.0,
                   rms_eps: float = 1e-6, round_bf16: bool = False) -> dict:
    """Gradients of L = sum(z_bar * z) for the RT layer on x [N][R][d] (naive schedule).

    round_bf16: the derivatives are taken at the forward values as a bf16 layer stores them.
    Returns float64 arrays by name: x, w_q, w_k, w_v, w_o, w_1, w_2, g_attn, g_mlp; with
    round_bf16 also "z_stored", the forward output as stored (float32, bf16 values).
    """
    from . import layer_forward  # the forward values (rt_oracle.c, IEEE double)
    from . import round_bf16 as _round

    keep = (lambda t: _round(t)) if round_bf16 else (lambda t: t)

    x = np.asarray(x, dtype=np.float32)
    N, R, d = x.shape
    H = n_heads
    dh = d // H
    W = {n: np.asarray(weights[n], dtype=np.float64) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    F = W["w_1"].shape[0]
    g_attn = np.ones(d) if weights.get("g_attn") is None else np.asarray(weights["g_attn"], dtype=np.float64)
    g_mlp = np.ones(d) if weights.get("g_mlp") is None else np.asarray(weights["g_mlp"], dtype=np.float64)
    rho, sigma, eps = residual_scale, softmax_scale, rms_eps

    fw = layer_forward(x, weights, n_heads=H, softmax_scale=sigma, residual_scale=rho, rms_eps=rms_eps,
                       round_bf16=round_bf16, want=("z", "k", "v", "q", "k_eph", "v_eph", "a", "h"))
    xd = x.astype(np.float64)
    z = fw["x_next"].astype(np.float64) if round_bf16 else fw["z"]   # the output as stored
    h, a = fw["h"], keep(fw["a"])
    heads = lambda t: t.reshape(N, R, H, dh)
    q, ke, ve, k, v = (heads(keep(fw[n])) for n in ("q", "k_eph", "v_eph", "k", "v"))
    a_h = heads(a)
    m, rh = _rms_fwd(h, g_mlp, eps)
    if round_bf16:
        u = keep((g_mlp * keep(h) * rh) @ W["w_1"].T)   # the product reads h as bf16, its rms exact
        m = keep(m)
    else:
        u = m @ W["w_1"].T                              # [N][R][F], pre-activation
    ux, _ = _rms_fwd(xd, g_attn, eps)
    uz, _ = _rms_fwd(z, g_attn, eps)
    ux, uz = keep(ux), keep(uz)
    gelu_u = keep(_gelu(u))

    zb = np.asarray(z_bar, dtype=np.float64)
    k_bar = np.zeros((N, R, H, dh))
    v_bar = np.zeros((N, R, H, dh))
    q_bar = np.zeros((N, R, H, dh))
    ke_bar = np.zeros((N, R, H, dh))
    ve_bar = np.zeros((N, R, H, dh))
    zt_bar = np.zeros((N, R, d))                          # z_bar(total) per position
    u_bar = np.zeros((N, R, F))
    h_bar = np.zeros((N, R, d))
    a_bar = np.zeros((N, R, d))
    g_attn_bar = np.zeros(d)
    g_mlp_bar = np.zeros(d)

    for t in reversed(range(N)):
        # the persistent pair of position t is complete: every query > t has been differentiated
        uz_bar = k_bar[t].reshape(R, d) @ W["w_k"] + v_bar[t].reshape(R, d) @ W["w_v"]
        dz, dg = _rms_bwd(z[t], g_attn, uz_bar, eps)
        g_attn_bar += dg
        zt_bar[t] = zb[t] + dz
        # MLP and output projection
        u_bar[t] = rho * (zt_bar[t] @ W["w_2"]) * _gelu_grad(u[t])
        dh_, dg = _rms_bwd(h[t], g_mlp, u_bar[t] @ W["w_1"], eps)
        g_mlp_bar += dg
        h_bar[t] = zt_bar[t] + dh_
        a_bar[t] = rho * (h_bar[t] @ W["w_o"])
        # attention of query t: persistent pairs 0..t-1 and the ephemeral pair
        ab = a_bar[t].reshape(R, H, dh)
        qt = q[t]
        s = sigma * np.concatenate([np.einsum("rhe,irhe->irh", qt, k[:t]),
                                    np.einsum("rhe,rhe->rh", qt, ke[t])[None]], axis=0)   # [t+1][R][H]
        p = np.exp(s - s.max(axis=0, keepdims=True))
        p /= p.sum(axis=0, keepdims=True)
        D = np.einsum("rhe,rhe->rh", ab, a_h[t])
        vals = np.concatenate([v[:t], ve[t][None]], axis=0)
        keys = np.concatenate([k[:t], ke[t][None]], axis=0)
        ds = p * (np.einsum("rhe,irhe->irh", ab, vals) - D[None])
        v_bar[:t] += p[:t, ..., None] * ab[None]
        k_bar[:t] += sigma * ds[:t, ..., None] * qt[None]
        ve_bar[t] = p[t][..., None] * ab
        ke_bar[t] = sigma * ds[t][..., None] * qt
        q_bar[t] = sigma * np.einsum("irh,irhe->rhe", ds, keys)

    flat = lambda t: t.reshape(N, R, d)
    ux_bar = flat(q_bar) @ W["w_q"] + flat(ke_bar) @ W["w_k"] + flat(ve_bar) @ W["w_v"]
    dx, dg = _rms_bwd(xd, g_attn, ux_bar, eps)
    g_attn_bar += dg
    outer = lambda A, B: np.einsum("nro,nri->oi", A, B)
    out = {
        "x": h_bar + dx,
        "w_q": outer(flat(q_bar), ux),
        "w_k": outer(flat(ke_bar), ux) + outer(flat(k_bar), uz),
        "w_v": outer(flat(ve_bar), ux) + outer(flat(v_bar), uz),
        "w_o": rho * outer(h_bar, a),
        "w_1": outer(u_bar, m),
        "w_2": rho * outer(zt_bar, gelu_u),
        "g_attn": g_attn_bar,
        "g_mlp": g_mlp_bar,
    }
    if round_bf16:
        out["z_stored"] = fw["x_next"]
    return out
