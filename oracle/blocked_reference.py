"""The blocked schedule of the RT layer in fp64 -- TEST INFRASTRUCTURE ONLY.

This is a second CPU implementation, following the algorithm of the
Recurrent Transformer reading note (lshu.cn/news/403416), summary section 4.2:
all queries are formed up front from the layer input; each query keeps an
online-softmax state (running maximum m, normaliser l, numerator o); when the
persistent pair of position t is revealed, the pairs t-b+1..t are merged into
the states of queries t+1..t+b (b = largest power of two dividing t). The state
merge of one block is the tile merge of IO-aware exact attention
(FlashAttention paragraph of the long-context survey translation,
blog.csdn.net/yorkhunter/article/details/138851205).

It exists only to pin the naive oracle: the note says the blocked algorithm is
exact, its output equal to the naive one up to the order of floating-point
operations. It is plain numpy in float64 and imports nothing from rt_oracle.c.
"""
from __future__ import annotations

import math

import numpy as np

from .schedule import step


def _rms(x, g, eps):
    return g * x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _gelu(u):
    erf = np.vectorize(math.erf)
    return 0.5 * u * (1.0 + erf(u / math.sqrt(2.0)))


class _State:
    """Online-softmax state of every query position, per row and head."""

    def __init__(self, n, rows, heads, dh):
        self.m = np.full((n, rows, heads), -np.inf)
        self.l = np.zeros((n, rows, heads))
        self.o = np.zeros((n, rows, heads, dh))

    def merge(self, j, q, K, V, sigma):
        """Merge pairs K, V [nb][rows][heads][dh] into query j's state; q [rows][heads][dh]."""
        s = sigma * np.einsum("rhe,brhe->brh", q, K)        # scores of the block
        m_new = np.maximum(self.m[j], s.max(axis=0))
        alpha = np.where(np.isneginf(self.m[j]), 0.0, np.exp(self.m[j] - m_new))
        p = np.exp(s - m_new[None])
        self.l[j] = alpha * self.l[j] + p.sum(axis=0)
        self.o[j] = alpha[..., None] * self.o[j] + np.einsum("brh,brhe->rhe", p, V)
        self.m[j] = m_new

    def finish(self, j, q, k_e, v_e, sigma):
        """Merge the ephemeral pair of query j and return o / l."""
        self.merge(j, q, k_e[None], v_e[None], sigma)
        return self.o[j] / self.l[j][..., None]


def attention(q, k_eph, v_eph, k, v, softmax_scale):
    """Blocked RT attention on given tensors [N][R][H][dh] (all pairs known up front)."""
    q, k_eph, v_eph, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k_eph, v_eph, k, v))
    n, rows, heads, dh = q.shape
    st = _State(n, rows, heads, dh)
    a = np.empty_like(q)
    for t in range(1, n + 1):
        a[t - 1] = st.finish(t - 1, q[t - 1], k_eph[t - 1], v_eph[t - 1], softmax_scale)
        (k0, k1), (q0, q1) = step(t, n)
        for j in range(q0, q1 + 1):
            st.merge(j - 1, q[j - 1], k[k0 - 1:k1], v[k0 - 1:k1], softmax_scale)
    return a


def layer_forward(x, w, *, n_heads, softmax_scale, residual_scale=1.0, rms_eps=1e-6, kv_from_input=False,
                  qk_norm=False, kv_source_norm=True):
    """Blocked-schedule RT layer in float64 on x [N][R][d]. Returns z, k, v (float64).
    qk_norm: queries and keys RMS-normalised per head (gains g_q, g_k).
    kv_source_norm=False: the persistent pair is W_{k,v} z_t, without the RMS."""
    x = np.asarray(x, dtype=np.float64)
    n, rows, d = x.shape
    dh = d // n_heads
    W = {k_: np.asarray(v_, dtype=np.float64) for k_, v_ in w.items()}
    g_attn = W.get("g_attn", np.ones(d))
    g_mlp = W.get("g_mlp", np.ones(d))
    # every query and ephemeral pair depends only on the input: formed up front
    u = _rms(x, g_attn, rms_eps)
    g_q = W.get("g_q", np.ones(d)).reshape(n_heads, dh)
    g_k = W.get("g_k", np.ones(d)).reshape(n_heads, dh)
    head_rms = (lambda y, g: _rms(y, g, rms_eps)) if qk_norm else (lambda y, g: y)
    q = head_rms((u @ W["w_q"].T).reshape(n, rows, n_heads, dh), g_q)
    k_eph = head_rms((u @ W["w_k"].T).reshape(n, rows, n_heads, dh), g_k)
    v_eph = (u @ W["w_v"].T).reshape(n, rows, n_heads, dh)
    K = np.zeros((n, rows, n_heads, dh))
    V = np.zeros((n, rows, n_heads, dh))
    z = np.zeros((n, rows, d))
    st = _State(n, rows, n_heads, dh)
    rho = residual_scale
    for t in range(1, n + 1):
        i = t - 1
        a = st.finish(i, q[i], k_eph[i], v_eph[i], softmax_scale).reshape(rows, d)
        h = x[i] + rho * a @ W["w_o"].T
        z[i] = h + rho * _gelu(_rms(h, g_mlp, rms_eps) @ W["w_1"].T) @ W["w_2"].T
        src = x[i] if kv_from_input else z[i]
        us = _rms(src, g_attn, rms_eps) if (kv_from_input or kv_source_norm) else src
        K[i] = head_rms((us @ W["w_k"].T).reshape(rows, n_heads, dh), g_k)
        V[i] = (us @ W["w_v"].T).reshape(rows, n_heads, dh)
        (k0, k1), (q0, q1) = step(t, n)
        for j in range(q0, q1 + 1):
            st.merge(j - 1, q[j - 1], K[k0 - 1:k1], V[k0 - 1:k1], softmax_scale)
    return {"z": z, "k": K.reshape(n, rows, d), "v": V.reshape(n, rows, d)}
