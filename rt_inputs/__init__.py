"""Seeded synthetic inputs for the Recurrent Transformer (RT) layer workloads.

This module is shared by the GPU library's tests, the bench and the CPU oracle.
It holds none of the layer's arithmetic: it only draws normal variates from
counter-free, per-tensor NumPy PCG64 streams and stores them in the requested
format (fp32, or bf16 by round-to-nearest-even via torch's cast).

Stream layout (stable, so any batch row can be regenerated on its own):
  * layer input x, batch row b:           SeedSequence(seed, spawn_key=(0, b)), shape [N][d]
  * weight j of layer l (j = 0..5 for
    W_q, W_k, W_v, W_o, W_1, W_2):         SeedSequence(seed, spawn_key=(1 + l, j)),
                                           N(0,1) scaled by 1/sqrt(d_in)
  * isolated-update tensor j (q, k', v',
    k, v for j = 0..4), batch row b:        SeedSequence(seed, spawn_key=(100 + j, b)), shape [N][H][dh]
Gains of both RMSNorms are vectors of ones.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "normal", "layer_input", "layer_weights",
    "attn_inputs", "to_storage",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes of one synthetic workload. Positions are 1..n_pos."""
    name: str
    batch: int
    n_pos: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ff: int
    n_layers: int
    dtype: str          # "f32" or "bf16": storage format of every tensor
    seed: int
    update_only: bool = False

    @property
    def tokens(self) -> int:
        return self.batch * self.n_pos


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", 2, 64, 64, 2, 32, 256, 1, "f32", 1000),
        Workload("update_b64_n4096", 64, 4096, 512, 8, 64, 0, 0, "bf16", 1001, update_only=True),
        Workload("layer_d768_b512_n1024", 512, 1024, 768, 12, 64, 3072, 1, "bf16", 1002),
        Workload("stack6_d1024_b512_n2048", 512, 2048, 1024, 16, 64, 4096, 6, "bf16", 1003),
        Workload("long_d1024_b8_n32768", 8, 32768, 1024, 16, 64, 4096, 1, "bf16", 1004),
    ]
}


def normal(seed: int, key: tuple, shape) -> np.ndarray:
    """N(0,1) draws in fp32 from the PCG64 stream named by (seed, key)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))
    return rng.standard_normal(shape, dtype=np.float32)


def to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Return the fp32 array of the values the storage format holds.

    For "bf16" every value is rounded to the nearest bf16 (ties to even) by
    torch's cast; the result is still an fp32 array (exactly representable).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype != "bf16":
        raise ValueError(f"unknown storage dtype {dtype!r}")
    import torch
    return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def layer_input(w: Workload, rows=None) -> np.ndarray:
    """Layer-1 input x as fp32 values of the storage format, shape [N][len(rows)][d]."""
    rows = list(range(w.batch)) if rows is None else [int(r) for r in rows]
    out = np.empty((w.n_pos, len(rows), w.d_model), dtype=np.float32)

    def fill(i):
        out[:, i, :] = to_storage(normal(w.seed, (0, rows[i]), (w.n_pos, w.d_model)), w.dtype)

    if len(rows) > 4:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(len(rows))))
    else:
        for i in range(len(rows)):
            fill(i)
    return out


def layer_weights(w: Workload, layer: int) -> dict:
    """Weights of one layer, row-major [out][in], N(0, 1/d_in), in the storage format."""
    d, f = w.d_model, w.d_ff
    shapes = [("w_q", d, d), ("w_k", d, d), ("w_v", d, d), ("w_o", d, d), ("w_1", f, d), ("w_2", d, f)]
    out = {}
    for j, (name, n_out, n_in) in enumerate(shapes):
        a = normal(w.seed, (1 + layer, j), (n_out, n_in)) * np.float32(1.0 / math.sqrt(n_in))
        out[name] = to_storage(a, w.dtype)
    out["g_attn"] = np.ones(d, dtype=np.float32)
    out["g_mlp"] = np.ones(d, dtype=np.float32)
    return out


def attn_inputs(w: Workload, rows=None) -> dict:
    """q, k', v' (ephemeral) and persistent k, v, each [N][len(rows)][H][dh], N(0,1)."""
    rows = list(range(w.batch)) if rows is None else [int(r) for r in rows]
    out = {}
    for j, name in enumerate(["q", "k_eph", "v_eph", "k", "v"]):
        a = np.empty((w.n_pos, len(rows), w.n_heads, w.head_dim), dtype=np.float32)
        for i, r in enumerate(rows):
            a[:, i] = to_storage(normal(w.seed, (100 + j, r), (w.n_pos, w.n_heads, w.head_dim)), w.dtype)
        out[name] = a
    return out
