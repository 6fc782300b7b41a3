"""CPU oracle for the Recurrent Transformer (RT) layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg use this
package. The GPU library (blocked_prefill_amd) never imports it, and this
package imports nothing from the library.

The arithmetic lives in rt_oracle.c (naive schedule, IEEE double); this module
marshals numpy arrays into it. layer_backward.py holds the layer's gradient
(the chain rule in numpy fp64 over rt_oracle.c's forward values). schedule.py holds the blocked schedule's integer
rules and blocked_reference.py the pages' blocked algorithm in fp64, which pins
the naive oracle (both are written from the Recurrent Transformer reading note,
lshu.cn/news/403416, summary section 4.2).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "librt_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)


class _Cfg(ctypes.Structure):
    _fields_ = [("n_pos", ctypes.c_int32), ("n_rows", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("softmax_scale", ctypes.c_double), ("residual_scale", ctypes.c_double),
                ("rms_eps", ctypes.c_double), ("kv_from_input", ctypes.c_int32),
                ("round_bf16", ctypes.c_int32), ("qk_norm", ctypes.c_int32), ("kv_source_norm", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [(n, _fp) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp", "g_q", "g_k")]


class _Out(ctypes.Structure):
    _fields_ = [(n, _dp) for n in ("z", "k", "v", "q", "k_eph", "v_eph", "a", "h", "g")] + [("x_next", _fp)]


def lib():
    """Load the oracle library, building it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.rto_round_bf16.restype = ctypes.c_double
        L.rto_round_bf16.argtypes = [ctypes.c_double]
        L.rto_num_threads.restype = ctypes.c_int
        L.rto_num_threads.argtypes = []
        L.rto_gelu.restype = ctypes.c_double
        L.rto_gelu.argtypes = [ctypes.c_double]
        L.rto_rmsnorm.restype = None
        L.rto_rmsnorm.argtypes = [_dp, ctypes.c_int, _fp, ctypes.c_double, _dp]
        L.rto_attention.restype = ctypes.c_int
        L.rto_attention.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double] + [_fp] * 5 + [_dp]
        L.rto_attention_at.restype = ctypes.c_int
        L.rto_attention_at.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double] + [_fp] * 5 + [
            ctypes.c_int, ctypes.POINTER(ctypes.c_int), _dp]
        L.rto_layer_forward.restype = ctypes.c_int
        L.rto_layer_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.POINTER(_Weights), _fp, ctypes.POINTER(_Out)]
        L.rto_attention_backward.argtypes = [ctypes.c_int] * 4 + [ctypes.c_double] + [_fp] * 6 + [_dp] * 5
        L.rto_attention_backward.restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    """Host threads the oracle uses."""
    return int(lib().rto_num_threads())


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_fp)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round each value (float64) to the nearest bf16, ties to even.

    The same definition as rto_round_bf16 in rt_oracle.c (8 significant bits,
    the binary32 exponent range with its subnormal spacing 2^-133, overflow to
    infinity), vectorised over the array.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                                   # a = f * 2^e, f in [0.5, 1)
    ulp_exp = np.maximum(e - 8, -133)
    r = np.ldexp(np.rint(np.ldexp(a, -ulp_exp)), ulp_exp)  # np.rint: ties to even
    r = np.where(r > np.ldexp(255.0, 120), np.inf, r)
    out = np.copysign(r, v)
    keep = (a == 0) | ~np.isfinite(v)
    return np.where(keep, v, out)


def round_bf16_scalar(x: float) -> float:
    """rto_round_bf16 of rt_oracle.c on one value."""
    return float(lib().rto_round_bf16(float(x)))


def gelu(u: np.ndarray) -> np.ndarray:
    f = lib().rto_gelu
    u = np.asarray(u, dtype=np.float64)
    return np.array([f(float(x)) for x in u.ravel()], dtype=np.float64).reshape(u.shape)


def rmsnorm(x: np.ndarray, g=None, eps: float = 1e-6) -> np.ndarray:
    """RMS normalisation of a 1-D vector with optional gain."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    g_arr, g_p = _f32(g) if g is not None else (None, ctypes.cast(None, _fp))
    lib().rto_rmsnorm(x.ctypes.data_as(_dp), x.size, g_p, eps, out.ctypes.data_as(_dp))
    return out


def attention(q, k_eph, v_eph, k, v, softmax_scale: float) -> np.ndarray:
    """Naive RT attention on given tensors [N][R][H][dh]; returns float64 a, same shape.

    Position t's query attends to persistent pairs 1..t-1 and its own
    ephemeral pair (summary sections 2.2 and 4.1 of the reading note).
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    N, R, H, dh = q.shape
    arrs = [_f32(t) for t in (q, k_eph, v_eph, k, v)]
    for a, _ in arrs:
        if a.shape != q.shape:
            raise ValueError("all attention tensors must share one shape")
    out = np.empty(q.shape, dtype=np.float64)
    st = lib().rto_attention(N, R, H, dh, softmax_scale, *[p for _, p in arrs], out.ctypes.data_as(_dp))
    if st != 0:
        raise RuntimeError(f"rto_attention failed with status {st}")
    return out


def attention_backward(q, k_eph, v_eph, k, v, a_bar, softmax_scale: float) -> dict:
    """Gradient of the naive RT attention map for the output adjoint a_bar = dL/da
    (all [N][R][H][dh]): returns float64 q, k_eph, v_eph, k, v gradients by name."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    arrs = [_f32(t) for t in (q, k_eph, v_eph, k, v, a_bar)]
    for a, _ in arrs:
        if a.shape != q.shape:
            raise ValueError("all attention tensors must share one shape")
    N, R, H, dh = q.shape
    outs = {n: np.empty(q.shape, dtype=np.float64) for n in ("q", "k_eph", "v_eph", "k", "v")}
    st = lib().rto_attention_backward(N, R, H, dh, softmax_scale, *[p for _, p in arrs],
                                      *[outs[n].ctypes.data_as(_dp) for n in ("q", "k_eph", "v_eph", "k", "v")])
    if st != 0:
        raise RuntimeError(f"rto_attention_backward failed with status {st}")
    return outs


def attention_at(q, k_eph, v_eph, k, v, softmax_scale: float, positions) -> np.ndarray:
    """Naive RT attention of the listed 1-based positions only; returns [len(positions)][R][H][dh] float64."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    N, R, H, dh = q.shape
    arrs = [_f32(t) for t in (q, k_eph, v_eph, k, v)]
    sel = np.ascontiguousarray(positions, dtype=np.int32)
    out = np.empty((len(sel), R, H, dh), dtype=np.float64)
    st = lib().rto_attention_at(N, R, H, dh, softmax_scale, *[p for _, p in arrs], len(sel),
                                sel.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), out.ctypes.data_as(_dp))
    if st != 0:
        raise RuntimeError(f"rto_attention_at failed with status {st}")
    return out


def layer_forward(x, weights: dict, *, n_heads: int, softmax_scale: float, residual_scale: float = 1.0,
                  rms_eps: float = 1e-6, kv_from_input: bool = False, round_bf16: bool = False,
                  qk_norm: bool = False, kv_source_norm: bool = True, want=("z", "k", "v")) -> dict:
    """Naive RT layer on x [N][R][d] (fp32 values). Returns float64 outputs by name.

    Names: z, k, v, q, k_eph, v_eph, a, h ([N][R][d]); g ([N][R][F]); and
    always x_next (float32, z as stored: the next layer's input).
    qk_norm: every query and key RMS-normalised per head (gains g_q, g_k of the
    weights, ones when absent).
    kv_source_norm: the persistent pair is W_{k,v} RMS_attn(z_t) (True) or
    W_{k,v} z_t (False, the literal reading of the cut formula).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    N, R, d = x.shape
    F = weights["w_1"].shape[0]
    if d % n_heads:
        raise ValueError("d_model must be a multiple of n_heads")
    cfg = _Cfg(N, R, d, n_heads, d // n_heads, F, softmax_scale, residual_scale, rms_eps,
               int(bool(kv_from_input)), int(bool(round_bf16)), int(bool(qk_norm)), int(bool(kv_source_norm)))
    keep = {}
    wp = {}
    for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp", "g_q", "g_k"):
        if weights.get(n) is None:
            wp[n] = ctypes.cast(None, _fp)
        else:
            keep[n], wp[n] = _f32(weights[n])
    W = _Weights(**wp)
    outs = {}
    op = {}
    for n in ("z", "k", "v", "q", "k_eph", "v_eph", "a", "h", "g"):
        if n in want:
            outs[n] = np.empty((N, R, F if n == "g" else d), dtype=np.float64)
            op[n] = outs[n].ctypes.data_as(_dp)
        else:
            op[n] = ctypes.cast(None, _dp)
    outs["x_next"] = np.empty((N, R, d), dtype=np.float32)
    op["x_next"] = outs["x_next"].ctypes.data_as(_fp)
    O = _Out(**op)
    st = lib().rto_layer_forward(ctypes.byref(cfg), ctypes.byref(W), x.ctypes.data_as(_fp), ctypes.byref(O))
    if st != 0:
        raise RuntimeError(f"rto_layer_forward failed with status {st}")
    return outs


def stack_forward(x, layers: list, **kw) -> list:
    """Layers applied in order, layer l+1 reading layer l's stored output. Returns each layer's outputs."""
    res = []
    cur = x
    for w in layers:
        o = layer_forward(cur, w, **kw)
        res.append(o)
        cur = o["x_next"]
    return res
