"""Host logic of bench.py (no GPU): the refusal of a multi-GPU run, and the
algorithmic byte and flop model of the blocked update that its roofline
divides by, pinned against closed forms of the schedule (each (key, query)
pair with key < query is visited once; the steps' blocks sum to (N/2)·log2 N
for N a power of two)."""
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_multi_gpu_run_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("n", [2, 3, 64, 300, 2048])
def test_update_flops_total_is_the_pair_count(n):
    """4*dh flops per visited (key, query) pair, N(N-1)/2 pairs, plus each
    finished query's ephemeral pair."""
    p, dh = 5, 64
    total = sum(bench.update_flops(t, n, p, dh) for t in range(1, n))
    assert total == 4 * dh * p * (n * (n - 1) // 2 + (n - 1))


@pytest.mark.parametrize("n", [2, 64, 2048])
def test_update_bytes_total_matches_the_closed_form(n):
    """N a power of two: every step's query block is whole, so with
    S = (N/2)·log2 N the KV blocks move 2·dh·s·S per pair, the queries dh·s·S,
    the state is read for S - (N-1) rows (not on a row's first touch, at
    t = 2^j) and written for S - (N-1) rows (not for the finished row), and
    every step reads the finished row's ephemeral pair and writes its output."""
    p, dh, s = 3, 64, 2
    S = n // 2 * int(math.log2(n))
    want = p * (2 * dh * s * S + dh * s * S + 2 * (dh + 2) * 4 * (S - (n - 1)) + 3 * dh * s * (n - 1))
    assert sum(bench.update_bytes(t, n, p, dh, s) for t in range(1, n)) == want


def test_update_bytes_at_the_stack_layer_shape():
    """B=512, 16 heads x 64, N=2048, bf16: 81.74 GB per layer, 39.93 MB per launch
    (9,978,000 bytes per (batch row, head) pair from the closed form above)."""
    p, n = 512 * 16, 2048
    total = sum(bench.update_bytes(t, n, p, 64, 2) for t in range(1, n))
    assert total == 81_739_776_000
    assert int(total / (n - 1)) == 39_931_497


def test_measured_traffic_belongs_to_its_workload():
    """The committed counters were taken on the stack's layer shape: no other
    workload reports them."""
    assert bench.measured_traffic("layer_d768_b512_n1024") is None
    assert bench.measured_traffic("long_d1024_b8_n32768") is None
