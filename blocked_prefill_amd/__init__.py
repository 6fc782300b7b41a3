"""Python binding of the MI355X Recurrent Transformer prefill library (librt_prefill.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/rt_prefill.h. Tensor arguments
may be torch device tensors (their data_ptr() is passed) or integer device
addresses. A missing library is an error: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "RT_F32", "RT_BF16", "RtError", "AttnDesc", "LayerDesc", "LayerWeights", "load", "library_path",
    "rt_blocked_attn_update", "rt_finalize_step", "rt_update_finalize_step", "rt_layer_workspace_bytes",
    "rt_layer_forward", "rt_layer_plan_create", "rt_layer_plan_launch", "rt_layer_plan_destroy", "rt_schedule_step",
    "rt_layer_decode_workspace_bytes", "rt_layer_decode_step", "rt_attn_forward", "rt_attn_backward",
    "rt_layer_backward_workspace_bytes", "rt_layer_backward", "LayerGrads", "rt_last_error", "EXPORTED",
    "rt_stack_workspace_bytes", "rt_stack_forward", "rt_stack_plan_create", "rt_layer_decode_step_static",
    "RT_DECODE_STATIC_SCRATCH_BYTES", "RT_FLAG_DEBUG_SYNC", "RT_FLAG_NAIVE_SCHEDULE", "RT_FLAG_TRANSFORMER", "RT_FLAG_QK_NORM",
]

RT_F32, RT_BF16 = 0, 1
RT_FLAG_DEBUG_SYNC = 1
RT_FLAG_NAIVE_SCHEDULE = 2
RT_FLAG_TRANSFORMER = 4
RT_FLAG_QK_NORM = 8
RT_DECODE_STATIC_SCRATCH_BYTES = 64 << 20  # rt_layer_decode_step_static's scratch (include/rt_prefill.h)
_STATUS = {0: "RT_OK", 1: "RT_ERR_INVALID_ARG", 2: "RT_ERR_UNSUPPORTED", 3: "RT_ERR_WORKSPACE", 4: "RT_ERR_HIP",
           5: "RT_ERR_INTERNAL"}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "librt_prefill.so")

# every symbol include/rt_prefill.h declares
EXPORTED = ["rt_blocked_attn_update", "rt_finalize_step", "rt_update_finalize_step", "rt_layer_workspace_bytes", "rt_layer_forward",
            "rt_layer_plan_create", "rt_layer_plan_launch", "rt_layer_plan_destroy", "rt_schedule_step",
            "rt_layer_decode_workspace_bytes", "rt_layer_decode_step", "rt_attn_forward", "rt_attn_backward",
            "rt_layer_backward_workspace_bytes", "rt_layer_backward", "rt_last_error",
            "rt_stack_workspace_bytes", "rt_stack_forward", "rt_stack_plan_create", "rt_layer_decode_step_static"]


class RtError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int), ("softmax_scale", ctypes.c_float)]


class LayerDesc(ctypes.Structure):
    _fields_ = [("attn", AttnDesc), ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("residual_scale", ctypes.c_float), ("kv_source_norm", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]

    def __init__(self, *args, kv_source_norm: int = 1, **kw):
        # 1 (the persistent pair reads RMS_attn(z_t)) unless the caller says otherwise
        super().__init__(*args, kv_source_norm=kv_source_norm, **kw)


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp", "g_q",
                                               "g_k")]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp")]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


def load():
    """Load librt_prefill.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(f"{library_path} is missing: build it first (python -m blocked_prefill_amd.build)")
        L = ctypes.CDLL(library_path)
        sig = {
            "rt_blocked_attn_update": [ctypes.POINTER(AttnDesc), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
            "rt_finalize_step": [ctypes.POINTER(AttnDesc), _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
            "rt_update_finalize_step": [ctypes.POINTER(AttnDesc), _i32] + [_vp] * 10,
            "rt_layer_forward": [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), _vp, _vp, _vp, _vp,
                                 _vp, ctypes.c_size_t, _vp],
            "rt_layer_plan_create": [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), _vp, _vp, _vp, _vp,
                                     _vp, ctypes.c_size_t, ctypes.POINTER(_vp)],
            "rt_layer_plan_launch": [_vp, _vp],
            "rt_attn_forward": [ctypes.POINTER(AttnDesc)] + [_vp] * 11,
            "rt_attn_backward": [ctypes.POINTER(AttnDesc)] + [_vp] * 15,
            "rt_layer_decode_step": [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), _i32, _vp, _vp, _vp,
                                     _vp, _vp, ctypes.c_size_t, _vp],
            "rt_layer_decode_step_static": [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), _i32, _vp,
                                            _vp, _vp, _vp, _vp],
            "rt_schedule_step": [_i32, _i32] + [ctypes.POINTER(_i32)] * 4,
            "rt_layer_backward": [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), _vp, _vp, _vp, _vp,
                                  ctypes.POINTER(LayerGrads), _vp, ctypes.c_size_t, _vp],
            "rt_stack_forward": [ctypes.POINTER(LayerDesc), _i32, ctypes.POINTER(LayerWeights), _vp,
                                 ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp, ctypes.c_size_t,
                                 _vp],
            "rt_stack_plan_create": [ctypes.POINTER(LayerDesc), _i32, ctypes.POINTER(LayerWeights), _vp,
                                     ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp), _vp,
                                     ctypes.c_size_t, ctypes.POINTER(_vp)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.rt_layer_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.rt_layer_workspace_bytes.restype = ctypes.c_size_t
        L.rt_layer_decode_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.rt_layer_decode_workspace_bytes.restype = ctypes.c_size_t
        L.rt_layer_backward_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.rt_layer_backward_workspace_bytes.restype = ctypes.c_size_t
        L.rt_stack_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), _i32]
        L.rt_stack_workspace_bytes.restype = ctypes.c_size_t
        L.rt_layer_plan_destroy.argtypes = [_vp]
        L.rt_layer_plan_destroy.restype = None
        L.rt_last_error.argtypes = []
        L.rt_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def rt_last_error() -> str:
    return load().rt_last_error().decode()


def _check(st: int):
    if st != 0:
        raise RtError(st, rt_last_error())


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def rt_schedule_step(t: int, n: int):
    """((kv_first, kv_last), (q_first, q_last)) of step t, 1-based inclusive."""
    o = [_i32() for _ in range(4)]
    _check(load().rt_schedule_step(t, n, *[ctypes.byref(v) for v in o]))
    return (o[0].value, o[1].value), (o[2].value, o[3].value)


def rt_blocked_attn_update(desc: AttnDesc, t: int, q, k, v, m, l, o, stream=None):
    _check(load().rt_blocked_attn_update(ctypes.byref(desc), t, _ptr(q), _ptr(k), _ptr(v), _ptr(m), _ptr(l),
                                         _ptr(o), _stream(stream)))


def rt_finalize_step(desc: AttnDesc, t: int, q, k_eph, v_eph, m, l, o, a_t, stream=None):
    _check(load().rt_finalize_step(ctypes.byref(desc), t, _ptr(q), _ptr(k_eph), _ptr(v_eph), _ptr(m), _ptr(l),
                                   _ptr(o), _ptr(a_t), _stream(stream)))


def rt_update_finalize_step(desc: AttnDesc, t: int, q, k_eph, v_eph, k, v, m, l, o, a_next, stream=None):
    _check(load().rt_update_finalize_step(ctypes.byref(desc), t, _ptr(q), _ptr(k_eph), _ptr(v_eph), _ptr(k), _ptr(v),
                                          _ptr(m), _ptr(l), _ptr(o), _ptr(a_next), _stream(stream)))


def rt_attn_forward(desc: AttnDesc, q, k_eph, v_eph, k, v, a, lse, m, l, o, stream=None):
    _check(load().rt_attn_forward(ctypes.byref(desc), *[_ptr(t) for t in (q, k_eph, v_eph, k, v, a, lse, m, l, o)],
                                  _stream(stream)))


def rt_attn_backward(desc: AttnDesc, q, k_eph, v_eph, k, v, a, lse, a_bar, q_bar, k_eph_bar, v_eph_bar, k_bar,
                     v_bar, delta, stream=None):
    _check(load().rt_attn_backward(ctypes.byref(desc), *[_ptr(t) for t in (
        q, k_eph, v_eph, k, v, a, lse, a_bar, q_bar, k_eph_bar, v_eph_bar, k_bar, v_bar, delta)], _stream(stream)))


def rt_layer_workspace_bytes(desc: LayerDesc) -> int:
    return int(load().rt_layer_workspace_bytes(ctypes.byref(desc)))


def _weights(w) -> LayerWeights:
    if isinstance(w, LayerWeights):
        return w
    return LayerWeights(**{n: _ptr(w.get(n)) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp",
                                                        "g_q", "g_k")})


def rt_layer_forward(desc: LayerDesc, weights, x, z, k_cache, v_cache, workspace, workspace_bytes=None,
                     stream=None):
    ws = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    W = _weights(weights)
    _check(load().rt_layer_forward(ctypes.byref(desc), ctypes.byref(W), _ptr(x), _ptr(z), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(workspace), ws, _stream(stream)))


def rt_layer_decode_workspace_bytes(desc: LayerDesc) -> int:
    return int(load().rt_layer_decode_workspace_bytes(ctypes.byref(desc)))


def rt_layer_decode_step(desc: LayerDesc, weights, n_past: int, x_t, z_t, k_cache, v_cache, workspace,
                         workspace_bytes=None, stream=None):
    ws = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    W = _weights(weights)
    _check(load().rt_layer_decode_step(ctypes.byref(desc), ctypes.byref(W), n_past, _ptr(x_t), _ptr(z_t),
                                       _ptr(k_cache), _ptr(v_cache), _ptr(workspace), ws, _stream(stream)))


def rt_layer_decode_step_static(desc: LayerDesc, weights, n_past: int, x_t, z_t, k_cache, v_cache, stream=None):
    """rt_layer_decode_step with the library's own static scratch (no workspace, no allocation)."""
    W = _weights(weights)
    _check(load().rt_layer_decode_step_static(ctypes.byref(desc), ctypes.byref(W), n_past, _ptr(x_t), _ptr(z_t),
                                              _ptr(k_cache), _ptr(v_cache), _stream(stream)))


def rt_layer_backward_workspace_bytes(desc: LayerDesc) -> int:
    return int(load().rt_layer_backward_workspace_bytes(ctypes.byref(desc)))


def rt_layer_backward(desc: LayerDesc, weights, x, z, z_bar, x_bar, grads, workspace, workspace_bytes=None,
                      stream=None):
    """grads: a LayerGrads or a dict of fp32 tensors by name (w_q .. w_2 required; g_attn, g_mlp optional)."""
    ws = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    W = _weights(weights)
    G = grads if isinstance(grads, LayerGrads) else LayerGrads(
        **{n: _ptr(grads.get(n)) for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2", "g_attn", "g_mlp")})
    _check(load().rt_layer_backward(ctypes.byref(desc), ctypes.byref(W), _ptr(x), _ptr(z), _ptr(z_bar), _ptr(x_bar),
                                    ctypes.byref(G), _ptr(workspace), ws, _stream(stream)))


class Plan:
    """A captured layer forward; launch() replays it, destroy() frees the graph."""

    def __init__(self, handle, keep):
        self.handle = handle
        self._keep = keep  # the tensors baked into the graph stay referenced

    def launch(self, stream=None):
        rt_layer_plan_launch(self, stream)

    def destroy(self):
        rt_layer_plan_destroy(self)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def rt_layer_plan_create(desc: LayerDesc, weights, x, z, k_cache, v_cache, workspace, workspace_bytes=None) -> Plan:
    ws = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    W = _weights(weights)
    h = _vp()
    _check(load().rt_layer_plan_create(ctypes.byref(desc), ctypes.byref(W), _ptr(x), _ptr(z), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(workspace), ws, ctypes.byref(h)))
    return Plan(h.value, (weights, x, z, k_cache, v_cache, workspace))


def rt_stack_workspace_bytes(desc: LayerDesc, n_layers: int) -> int:
    return int(load().rt_stack_workspace_bytes(ctypes.byref(desc), n_layers))


def _stack_args(weights, z, k_cache, v_cache):
    n = len(weights)
    if not (len(z) == len(k_cache) == len(v_cache) == n):
        raise ValueError("weights, z, k_cache and v_cache need one entry per layer")
    W = (LayerWeights * n)(*[_weights(w) for w in weights])
    arr = lambda ts: (_vp * n)(*[_ptr(t) for t in ts])  # noqa: E731
    return n, W, arr(z), arr(k_cache), arr(v_cache)


def rt_stack_forward(desc: LayerDesc, weights, x, z, k_cache, v_cache, workspace, workspace_bytes=None,
                     stream=None):
    """weights, z, k_cache, v_cache: one entry per layer (z[l] is layer l+1's input)."""
    ws = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    n, W, Z, K, V = _stack_args(weights, z, k_cache, v_cache)
    _check(load().rt_stack_forward(ctypes.byref(desc), n, W, _ptr(x), Z, K, V, _ptr(workspace), ws,
                                   _stream(stream)))


def rt_stack_plan_create(desc: LayerDesc, weights, x, z, k_cache, v_cache, workspace, workspace_bytes=None) -> Plan:
    ws = workspace_bytes if workspace_bytes is not None else workspace.numel() * workspace.element_size()
    n, W, Z, K, V = _stack_args(weights, z, k_cache, v_cache)
    h = _vp()
    _check(load().rt_stack_plan_create(ctypes.byref(desc), n, W, _ptr(x), Z, K, V, _ptr(workspace), ws,
                                       ctypes.byref(h)))
    return Plan(h.value, (weights, x, z, k_cache, v_cache, workspace))


def rt_layer_plan_launch(plan: Plan, stream=None):
    _check(load().rt_layer_plan_launch(plan.handle, _stream(stream)))


def rt_layer_plan_destroy(plan: Plan):
    if plan.handle:
        load().rt_layer_plan_destroy(plan.handle)
        plan.handle = None
