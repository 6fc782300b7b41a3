"""The allocation-free decode entry point (rt_layer_decode_step_static) against
rt_layer_decode_step, through the C ABI: the same kernels on the same inputs,
so every output must be bit-identical. Two calls in a row, the second on a
smaller input (fewer batch rows, a shorter cache) than the first, since the
static scratch keeps the previous call's contents; and a shape whose scratch
exceeds the static array is refused before any launch."""
import math

import numpy as np
import pytest

import blocked_prefill_amd as rt
import rt_inputs
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.ensure_built()


def _weights(seed, d, f):
    rng = np.random.default_rng(seed)
    w = {
        "w_q": rng.standard_normal((d, d)) / math.sqrt(d), "w_k": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_v": rng.standard_normal((d, d)) / math.sqrt(d), "w_o": rng.standard_normal((d, d)) / math.sqrt(d),
        "w_1": rng.standard_normal((f, d)) / math.sqrt(d), "w_2": rng.standard_normal((d, f)) / math.sqrt(f),
    }
    w = {k: G.dev(rt_inputs.to_storage(v.astype(np.float32), "bf16"), "bf16") for k, v in w.items()}
    w["g_attn"] = G.dev((1 + 0.2 * rng.standard_normal(d)).astype(np.float32), "f32")
    w["g_mlp"] = G.dev((1 + 0.2 * rng.standard_normal(d)).astype(np.float32), "f32")
    return w


def _case(b, n_past, d, h, f, seed):
    """A prefill of n_past positions into caches of capacity n_past + 1, then position n_past + 1
    decoded twice: through rt_layer_decode_step (workspace) and rt_layer_decode_step_static,
    each into its own copy of the caches."""
    import torch
    n = n_past + 1
    x = G.dev(rt_inputs.to_storage(np.random.default_rng(seed).standard_normal((n, b, d)).astype(np.float32),
                                   "bf16"), "bf16")
    w = _weights(seed + 1, d, f)
    desc = G.layer_desc(b, n, d, h, f, "bf16", 1.0 / math.sqrt(d // h))
    kc = torch.zeros((n, b, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    if n_past:
        pre = G.layer_desc(b, n_past, d, h, f, "bf16", 1.0 / math.sqrt(d // h))
        ws = torch.empty(rt.rt_layer_workspace_bytes(pre), dtype=torch.uint8, device="cuda")
        z_pre = torch.empty((n_past, b, d), dtype=torch.bfloat16, device="cuda")
        rt.rt_layer_forward(pre, w, x[:n_past], z_pre, kc[:n_past], vc[:n_past], ws)
    kc2, vc2 = kc.clone(), vc.clone()
    z1 = torch.full((b, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    z2 = torch.full_like(z1, float("nan"))
    ws = torch.empty(rt.rt_layer_decode_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
    rt.rt_layer_decode_step(desc, w, n_past, x[n_past], z1, kc, vc, ws)
    rt.rt_layer_decode_step_static(desc, w, n_past, x[n_past], z2, kc2, vc2)
    torch.cuda.synchronize()
    return (z1, kc, vc), (z2, kc2, vc2)


def test_static_decode_equals_the_workspace_decode_on_two_calls_in_a_row():
    import torch
    for b, n_past, seed in ((24, 70, 3), (5, 17, 9)):  # the second call smaller than the first
        (z1, k1, v1), (z2, k2, v2) = _case(b, n_past, 256, 4, 512, seed)
        assert bool(torch.isfinite(z2).all())
        for name, a, c in (("z", z1, z2), ("k_cache", k1, k2), ("v_cache", v1, v2)):
            assert torch.equal(a, c), f"B={b} n_past={n_past}: {name} differs"


def test_static_decode_refuses_a_shape_beyond_its_scratch():
    # B=4096, d=1024, F=4096 with gains needs more than the static array
    desc = G.layer_desc(4096, 8, 1024, 16, 4096, "bf16", 0.125)
    assert rt.rt_layer_decode_workspace_bytes(desc) > rt.RT_DECODE_STATIC_SCRATCH_BYTES
    fake = 1 << 20
    W = {n: fake for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_decode_step_static(desc, W, 3, fake, fake, fake, fake)
    assert e.value.status == 3 and "static" in str(e.value)
