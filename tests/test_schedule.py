"""Pins of the blocked schedule's integer rules (oracle side, CPU only).

Recurrent Transformer reading note (lshu.cn/news/403416), summary section 4.2:
block size = largest power of two dividing t; the note's worked example;
every pair (s < j) is applied exactly once (the algorithm is exact); the work
is Theta(N log N) pairs-of-positions touched, O(log N) per step on average.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import schedule

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_from_the_note():
    g = json.load(open(os.path.join(GOLDEN, "schedule_worked_example.json")))
    (k0, k1), (q0, q1) = schedule.step(g["t"], 1 << 20)
    assert schedule.block_size(g["t"]) == g["block_size"]
    assert [q0, q1] == g["query_positions"]
    assert [k0, k1] == g["kv_positions"]


def test_block_size_is_largest_power_of_two_divisor():
    for t in range(1, 1 << 16):
        b = schedule.block_size(t)
        assert b & (b - 1) == 0 and t % b == 0 and (t // b) % 2 == 1
    with pytest.raises(ValueError):
        schedule.block_size(0)


@pytest.mark.parametrize("n", list(range(1, 70)) + [100, 127, 128, 129, 200, 255, 256, 300])
def test_every_causal_pair_covered_exactly_once(n):
    c = schedule.coverage(n)
    expect = np.triu(np.ones((n, n), dtype=np.int64), k=1)  # C[s, j] = 1 iff s < j
    assert np.array_equal(c, expect)


def _interval_check(n):
    """O(N log N) version: the KV blocks applied to query j tile [1, j-1] with no overlap."""
    got = [[] for _ in range(n + 1)]
    for t in range(1, n):
        (k0, k1), (q0, q1) = schedule.step(t, n)
        for j in range(q0, q1 + 1):
            got[j].append((k0, k1))
    for j in range(1, n + 1):
        iv = sorted(got[j])
        nxt = 1
        for a, b in iv:
            assert a == nxt, (n, j, iv)
            nxt = b + 1
        assert nxt == j, (n, j, iv)


@pytest.mark.parametrize("n", [1000, 1024, 4096, 5000, 32768])
def test_coverage_large_n_interval_check(n):
    _interval_check(n)


@pytest.mark.parametrize("k", range(1, 16))
def test_work_closed_forms_power_of_two(k):
    n = 1 << k
    sum_b = sum(schedule.block_size(t) for t in range(1, n))
    pairs = sum(schedule.block_size(t) * (schedule.step(t, n)[1][1] - t) for t in range(1, n))
    assert sum_b == (n // 2) * k                 # Theta(N log N) positions touched
    assert pairs == n * (n - 1) // 2             # exactly the causal pair count
    lv = schedule.level_counts(n)
    for i in range(k):
        assert lv[1 << i] == n >> (i + 1)        # steps at level 2^i


def test_positions_touched_per_step_is_logarithmic_on_average():
    for k in (10, 11, 15):
        n = 1 << k
        avg = sum(schedule.block_size(t) for t in range(1, n)) / (n - 1)
        assert abs(avg - math.log2(n) / 2 * n / (n - 1)) < 1e-12
