"""The C-ABI library loads, exports what include/rt_prefill.h declares, and its
host-side logic (schedule rule, argument validation, workspace sizing) behaves
as documented -- all without a GPU (no call here reaches a HIP launch)."""
import ctypes
import os
import re

import pytest

import blocked_prefill_amd as rt
from oracle import schedule

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rt.library_path):
        from blocked_prefill_amd import build
        build.build()
    return rt.load()


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(rt_[a-z_0-9]+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported(lib):
    declared = _declared_functions()
    assert declared, "no declarations found"
    assert declared == set(rt.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_library_is_hip_code_for_gfx950(lib):
    blob = open(rt.library_path, "rb").read()
    assert b"gfx950" in blob


def test_host_schedule_matches_the_pages_rule(lib):
    for n in (1, 2, 3, 7, 64, 100, 4096, 32768):
        for t in list(range(1, min(n, 300) + 1)) + [n]:
            assert rt.rt_schedule_step(t, n) == schedule.step(t, n), (t, n)


def test_host_schedule_rejects_out_of_range(lib):
    for t, n in [(0, 4), (5, 4), (1, 0), (-1, 8)]:
        with pytest.raises(rt.RtError) as e:
            rt.rt_schedule_step(t, n)
        assert e.value.status == 1


def _attn(**kw):
    d = dict(batch=2, seq_len=16, n_heads=2, head_dim=64, dtype=rt.RT_BF16, softmax_scale=0.125)
    d.update(kw)
    return rt.AttnDesc(**d)


def _layer(**kw):
    a = kw.pop("attn", _attn())
    d = dict(attn=a, d_model=a.n_heads * a.head_dim, d_ff=256, rms_eps=1e-6, residual_scale=1.0, flags=0)
    d.update(kw)
    return rt.LayerDesc(**d)


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (validation fails first)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), 1), (dict(seq_len=-3), 1), (dict(head_dim=48), 2), (dict(head_dim=256), 2),
    (dict(dtype=7), 1), (dict(softmax_scale=float("inf")), 1), (dict(softmax_scale=-0.5), 1),
])
def test_update_rejects_bad_descriptors(lib, kw, status):
    with pytest.raises(rt.RtError) as e:
        rt.rt_blocked_attn_update(_attn(**kw), 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == status


def test_update_rejects_bad_step_and_pointers(lib):
    d = _attn()
    for t in (0, 17):
        with pytest.raises(rt.RtError) as e:
            rt.rt_blocked_attn_update(d, t, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
        assert e.value.status == 1 and "t=" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_blocked_attn_update(d, 3, FAKE, None, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert "k is NULL" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_blocked_attn_update(d, 3, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    assert "aligned" in str(e.value)


def test_update_at_last_position_is_a_noop(lib):
    # t = N has no query left: valid, returns before any launch
    rt.rt_blocked_attn_update(_attn(seq_len=16), 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)


def test_attention_forward_and_backward_reject_bad_arguments(lib):
    d = _attn()
    args = [FAKE] * 10
    with pytest.raises(rt.RtError) as e:
        rt.rt_attn_forward(d, *args[:6], None, *args[7:], stream=0)
    assert "lse is NULL" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_attn_forward(d, FAKE + 8, *args[1:], stream=0)
    assert "aligned" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_attn_backward(d, *([FAKE] * 13), None, stream=0)
    assert "delta is NULL" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_attn_backward(_attn(head_dim=48), *([FAKE] * 14), stream=0)
    assert e.value.status == 2


def test_finalize_rejects_bad_arguments(lib):
    d = _attn()
    with pytest.raises(rt.RtError):
        rt.rt_finalize_step(d, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0)
    with pytest.raises(rt.RtError) as e:
        rt.rt_finalize_step(d, 2, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, stream=0)
    assert "state" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_finalize_step(d, 1, FAKE, FAKE, FAKE, None, None, None, None, stream=0)
    assert "a_t is NULL" in str(e.value)


def test_workspace_bytes(lib):
    d = _layer()
    n, b, h, dh, f = 16, 2, 2, 64, 256
    D = h * dh
    al = lambda x: (x + 255) // 256 * 256
    want = 3 * al(n * b * D * 2) + 2 * al(n * b * h * 4) + al(n * b * D * 4) + al(b * D * 2) + al(b * D * 4) \
        + al(b * f * 2) + al(b * D * 2) + 2 * al(D // 32 * b * 4 + 4) \
        + 3 * al(2 * D * D * 2) + al(2 * f * D * 2) \
        + al(n * b * 16)  # gain-folded bf16 weights (two halves per row); quarter-row sums of x^2
    assert rt.rt_layer_workspace_bytes(d) == want
    assert rt.rt_layer_workspace_bytes(_layer(d_model=100)) == 0
    assert rt.rt_layer_workspace_bytes(_layer(d_ff=100)) == 0  # bf16 needs multiples of 128


def test_workspace_bytes_of_the_other_modes(lib):
    n, b, h, dh, f = 16, 2, 2, 64, 256
    D = h * dh
    al = lambda x: (x + 255) // 256 * 256
    weights = 3 * al(2 * D * D * 2) + al(2 * f * D * 2)  # gain-folded bf16 weights, two halves per row
    xss = lambda rows: al(rows * 16)  # quarter-row sums of x^2 for the up-front projection

    def tail(rows):  # a, h, g, hb, hss, zss
        return al(rows * D * 2) + al(rows * D * 4) + al(rows * f * 2) + al(rows * D * 2) \
            + 2 * al(D // 32 * rows * 4 + 4)
    # naive schedule: no online-softmax state
    naive = 3 * al(n * b * D * 2) + tail(b) + weights + xss(n * b)
    assert rt.rt_layer_workspace_bytes(_layer(flags=rt.RT_FLAG_NAIVE_SCHEDULE)) == naive
    # Transformer: queries only (pairs go to the caches), every buffer over N*B rows
    tf = al(n * b * D * 2) + tail(n * b) + weights + xss(n * b)
    assert rt.rt_layer_workspace_bytes(_layer(flags=rt.RT_FLAG_TRANSFORMER)) == tf
    # decode: one position, independent of seq_len and of the flags
    dec = 3 * al(b * D * 2) + tail(b) + weights + xss(b)
    for flags in (0, rt.RT_FLAG_TRANSFORMER, rt.RT_FLAG_NAIVE_SCHEDULE):
        assert rt.rt_layer_decode_workspace_bytes(_layer(flags=flags)) == dec
    assert rt.rt_layer_decode_workspace_bytes(_layer(attn=_attn(seq_len=4096))) == dec
    both = rt.RT_FLAG_NAIVE_SCHEDULE | rt.RT_FLAG_TRANSFORMER
    assert rt.rt_layer_workspace_bytes(_layer(flags=both)) == 0
    assert rt.rt_layer_workspace_bytes(_layer(flags=64)) == 0


def test_flags_are_validated(lib):
    W = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    for flags, text in ((rt.RT_FLAG_NAIVE_SCHEDULE | rt.RT_FLAG_TRANSFORMER, "exclude"), (64, "unknown flags")):
        with pytest.raises(rt.RtError) as e:
            rt.rt_layer_forward(_layer(flags=flags), W, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)
        assert e.value.status == 1 and text in str(e.value)
    # the bf16 query/key norm works within one 64-column tile: head_dim up to 64
    wide = _layer(attn=_attn(n_heads=1, head_dim=128), flags=rt.RT_FLAG_QK_NORM)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_forward(wide, W, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.status == 2 and "head_dim" in str(e.value)
    assert rt.rt_layer_workspace_bytes(_layer(flags=rt.RT_FLAG_QK_NORM)) == rt.rt_layer_workspace_bytes(_layer())
    with pytest.raises(rt.RtError) as e:  # gains must be aligned like the other gains
        rt.rt_layer_forward(_layer(flags=rt.RT_FLAG_QK_NORM), dict(W, g_q=FAKE + 4), FAKE, FAKE, FAKE, FAKE, FAKE,
                            1 << 30, stream=0)
    assert "aligned" in str(e.value)


def test_kv_source_norm_is_validated(lib):
    W = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    assert _layer().kv_source_norm == 1  # the binding's default: the persistent pair reads RMS_attn(z)
    lit = _layer(kv_source_norm=0)
    assert rt.rt_layer_workspace_bytes(lit) == rt.rt_layer_workspace_bytes(_layer())
    for bad, text in ((_layer(kv_source_norm=2), "0 or 1"),
                      (_layer(kv_source_norm=0, flags=rt.RT_FLAG_TRANSFORMER), "ephemeral")):
        assert rt.rt_layer_workspace_bytes(bad) == 0
        with pytest.raises(rt.RtError) as e:
            rt.rt_layer_forward(bad, W, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)
        assert e.value.status == 1 and text in str(e.value)
    G = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    assert rt.rt_layer_backward_workspace_bytes(lit) == 0
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_backward(lit, W, FAKE, FAKE, FAKE, FAKE, G, FAKE, 1 << 30, stream=0)
    assert e.value.status == 2


def test_decode_rejects_bad_arguments(lib):
    d = _layer()
    W = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    need = rt.rt_layer_decode_workspace_bytes(d)
    for n_past in (-1, 16, 17):  # seq_len 16 is the caches' capacity
        with pytest.raises(rt.RtError) as e:
            rt.rt_layer_decode_step(d, W, n_past, FAKE, FAKE, FAKE, FAKE, FAKE, need, stream=0)
        assert e.value.status == 1 and "n_past" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_decode_step(d, W, 3, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, stream=0)
    assert e.value.status == 3
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_decode_step(d, W, 3, FAKE, None, FAKE, FAKE, FAKE, need, stream=0)
    assert "z is NULL" in str(e.value)


def test_layer_rejects_bad_arguments(lib):
    d = _layer()
    W = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    need = rt.rt_layer_workspace_bytes(d)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_forward(d, W, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, stream=0)
    assert e.value.status == 3
    W2 = dict(W, w_o=None)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_forward(d, W2, FAKE, FAKE, FAKE, FAKE, FAKE, need, stream=0)
    assert "w_o is NULL" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_forward(d, W, FAKE, FAKE, FAKE, FAKE, FAKE + 16, need, stream=0)
    assert "256-byte" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_forward(_layer(d_model=64), W, FAKE, FAKE, FAKE, FAKE, FAKE, need, stream=0)
    assert e.value.status == 1
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_plan_create(_layer(rms_eps=-1.0), W, FAKE, FAKE, FAKE, FAKE, FAKE, need)
    assert e.value.status == 1


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    import importlib
    mod = importlib.reload(rt)
    monkeypatch.setattr(mod, "library_path", str(tmp_path / "absent.so"))
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        mod.load()
    importlib.reload(rt)


def test_layer_backward_validates_its_arguments(lib):
    d = _layer()
    W = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    G = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    need = rt.rt_layer_backward_workspace_bytes(d)
    assert need > rt.rt_layer_workspace_bytes(d)
    # the naive schedule is the same layer map; the Transformer layer and the query/key norm are not covered
    assert rt.rt_layer_backward_workspace_bytes(_layer(flags=rt.RT_FLAG_NAIVE_SCHEDULE)) == need
    for flags in (rt.RT_FLAG_TRANSFORMER, rt.RT_FLAG_QK_NORM):
        assert rt.rt_layer_backward_workspace_bytes(_layer(flags=flags)) == 0
        with pytest.raises(rt.RtError) as e:
            rt.rt_layer_backward(_layer(flags=flags), W, FAKE, FAKE, FAKE, FAKE, G, FAKE, need, stream=0)
        assert e.value.status == 2
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_backward(d, W, FAKE, FAKE, FAKE, FAKE, G, FAKE, need - 1, stream=0)
    assert e.value.status == 3
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_backward(d, W, FAKE, FAKE, None, FAKE, G, FAKE, need, stream=0)
    assert "z_bar is NULL" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_backward(d, W, FAKE, FAKE, FAKE, FAKE, dict(G, w_2=None), FAKE, need, stream=0)
    assert "grads->w_2 is NULL" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_backward(d, W, FAKE, FAKE, FAKE, FAKE, dict(G, g_mlp=FAKE + 2), FAKE, need, stream=0)
    assert "gain gradients" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_layer_backward(d, W, FAKE, FAKE, FAKE, FAKE, G, FAKE + 16, need, stream=0)
    assert "256-byte" in str(e.value)


def test_stack_workspace_and_arguments(lib):
    d = _layer()
    one = rt.rt_layer_workspace_bytes(d)
    for n in (1, 2, 6):
        assert rt.rt_stack_workspace_bytes(d, n) == n * one
    assert rt.rt_stack_workspace_bytes(d, 0) == 0
    assert rt.rt_stack_workspace_bytes(d, 1025) == 0
    assert rt.rt_stack_workspace_bytes(_layer(d_model=100), 2) == 0
    W = {n: FAKE for n in ("w_q", "w_k", "w_v", "w_o", "w_1", "w_2")}
    need = rt.rt_stack_workspace_bytes(d, 2)
    with pytest.raises(rt.RtError) as e:
        rt.rt_stack_forward(d, [W, W], FAKE, [FAKE, FAKE], [FAKE, FAKE], [FAKE, FAKE], FAKE, need - 1, stream=0)
    assert e.value.status == 3
    with pytest.raises(rt.RtError) as e:  # layer 1's weights
        rt.rt_stack_forward(d, [W, dict(W, w_1=None)], FAKE, [FAKE, FAKE], [FAKE, FAKE], [FAKE, FAKE], FAKE, need,
                            stream=0)
    assert e.value.status == 1 and "layer 1" in str(e.value) and "w_1 is NULL" in str(e.value)
    with pytest.raises(rt.RtError) as e:  # layer 1's input is layer 0's output
        rt.rt_stack_forward(d, [W, W], FAKE, [FAKE + 8, FAKE], [FAKE, FAKE], [FAKE, FAKE], FAKE, need, stream=0)
    assert "layer 0" in str(e.value) and "aligned" in str(e.value)
    with pytest.raises(rt.RtError) as e:
        rt.rt_stack_plan_create(d, [W, W], FAKE, [FAKE, FAKE], [FAKE, None], [FAKE, FAKE], FAKE, need)
    assert e.value.status == 1 and "k_cache is NULL" in str(e.value)
    with pytest.raises(ValueError):
        rt.rt_stack_forward(d, [W, W], FAKE, [FAKE], [FAKE, FAKE], [FAKE, FAKE], FAKE, need, stream=0)
    with pytest.raises(rt.RtError) as e:
        rt.rt_stack_forward(d, [], FAKE, [], [], [], FAKE, need, stream=0)
    assert e.value.status == 1 and "n_layers" in str(e.value)
