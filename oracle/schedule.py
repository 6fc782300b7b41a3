"""Integer rules of the blocked schedule -- TEST INFRASTRUCTURE ONLY.

Recurrent Transformer reading note (lshu.cn/news/403416), summary section 4.2
("blocked schedule"): when the persistent pair of position t is revealed, the
block of pairs ending at t is applied to the accumulators of a block of future
queries, the block size being the largest power of two that divides t. The
note's own example: once (k_4, v_4) exists, the accumulators of a_5..a_8 are
updated. Positions are 1-based. For a sequence of N positions the query block
is clipped at N (the pages only use powers of two; clipping is the plain
reading for other N).
"""
from __future__ import annotations

import numpy as np


def block_size(t: int) -> int:
    """Largest power of two dividing t (t >= 1)."""
    if t < 1:
        raise ValueError("positions start at 1")
    b = 1
    while t % (2 * b) == 0:
        b *= 2
    return b


def step(t: int, n: int):
    """Ranges (inclusive, 1-based) touched when pair t is revealed in a length-n sequence.

    Returns ((kv_first, kv_last), (q_first, q_last)); the query range is empty
    (q_first > q_last) when t + 1 > n.
    """
    b = block_size(t)
    return (t - b + 1, t), (t + 1, min(t + b, n))


def coverage(n: int) -> np.ndarray:
    """C[s, j] = number of steps that apply pair s (1..n) to query j (1..n), brute force."""
    c = np.zeros((n + 1, n + 1), dtype=np.int64)
    for t in range(1, n + 1):
        (k0, k1), (q0, q1) = step(t, n)
        for s in range(k0, k1 + 1):
            for j in range(q0, q1 + 1):
                c[s, j] += 1
    return c[1:, 1:]


def level_counts(n: int) -> dict:
    """Number of steps per block size, for steps 1..n-1 that touch at least one query."""
    out = {}
    for t in range(1, n):
        b = block_size(t)
        out[b] = out.get(b, 0) + 1
    return out
