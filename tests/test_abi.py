"""The C-ABI library: it loads, exports every function the header declares,
and its host-side checks reject bad arguments before anything is enqueued.
CPU only: no call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import moe_layer_gating_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_gfx950.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(moe.LIB_PATH):
        import moe_layer_gating_amd._build as b

        b.build()
    return moe.lib()


def test_header_declares_the_six_entry_points():
    names = _declared_functions()
    for n in ("moe_topk_gating", "moe_align_sort", "moe_grouped_gemm_w13_swiglu",
              "moe_grouped_gemm_w2", "moe_combine", "moe_fused_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name
        assert name in moe.EXPORTS


def test_status_strings(L):
    for rc in (0, -1, -2, -3, -4):
        assert L.moe_status_string(rc)
    assert L.moe_status_string(-99) == b"unknown status"


@pytest.mark.parametrize("shape,want", [
    ((16, 128, 8, 2, 256, 0), 0),
    ((8, 4096, 8, 2, 14336, 1), 0),
    ((4096, 7168, 256, 8, 2048, 2), 0),
    ((0, 128, 8, 2, 256, 2), 0),          # T = 0 is valid (a no-op)
    ((-1, 128, 8, 2, 256, 0), -1),
    ((4, 128, 0, 1, 256, 0), -1),         # E = 0
    ((4, 128, 1025, 2, 256, 0), -1),      # E > 1024
    ((4, 128, 8, 0, 256, 0), -1),         # k = 0
    ((4, 128, 8, 9, 256, 0), -1),         # k > E
    ((4, 128, 32, 17, 256, 0), -1),       # k > 16
    ((4, 128, 8, 2, 256, 3), -1),         # bad dtype
    ((4, 100, 8, 2, 256, 0), -2),         # H not a multiple of 128
    ((4, 128, 8, 2, 200, 1), -2),         # I not a multiple of 128
])
def test_check_shape(L, shape, want):
    T, H, E, k, I, dt = shape
    s = moe.make_shape(T, H, E, k, I, dt)
    assert moe.moe_check_shape(s) == want
    ws = moe.moe_workspace_bytes(s)
    assert (ws > 0) == (want == 0)


def test_align_sort_workspace_bytes(L):
    assert moe.moe_align_sort_workspace_bytes(4, 2, 8) > 0
    assert moe.moe_align_sort_workspace_bytes(4, 9, 8) == 0  # k > E
    assert moe.moe_align_sort_workspace_bytes(-1, 2, 8) == 0
    small = moe.moe_align_sort_workspace_bytes(1024, 8, 256)   # 8192 pairs: chunked sort
    big = moe.moe_align_sort_workspace_bytes(4096, 8, 256)
    assert 0 < small < big and big % 256 == 0


def test_workspace_routing_offsets(L):
    """The routing arrays of a fused call sit inside the workspace, 256-byte
    aligned, without overlapping one another, and depend only on T, E, k."""
    for T, E, k in ((1, 64, 8), (8, 8, 2), (4096, 256, 8), (17, 1024, 16)):
        s = moe.make_shape(T, 7168, E, k, 2048, 2)
        r = moe.moe_workspace_routing(s)
        total = moe.moe_workspace_bytes(s)
        regions = sorted([(r.topk_ids, T * k * 4), (r.topk_weights, T * k * 4),
                          (r.expert_counts, E * 4), (r.expert_offsets, (E + 1) * 4),
                          (r.sorted_ids, T * k * 4), (r.inv_perm, T * k * 4)])
        for (a, n), (b, _) in zip(regions, regions[1:]):
            assert a % 256 == 0 and a + n <= b
        assert regions[-1][0] + regions[-1][1] <= total
        r2 = moe.moe_workspace_routing(moe.make_shape(T, 128, E, k, 128, 0))
        assert [getattr(r, f) for f, _ in r._fields_] == [getattr(r2, f) for f, _ in r2._fields_]
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_routing(moe.make_shape(4, 100, 8, 2, 256, 0))


def test_workspace_grows_with_tokens(L):
    a = moe.moe_workspace_bytes(moe.make_shape(1, 4096, 64, 8, 8192, 2))
    b = moe.moe_workspace_bytes(moe.make_shape(16, 4096, 64, 8, 8192, 2))
    assert 0 < a < b
    assert a % 256 == 0 and b % 256 == 0


def _fake(addr):
    return ctypes.c_void_p(addr)


def test_invalid_pointers_rejected_before_launch(L):
    good = _fake(0x100000)
    odd = _fake(0x100004)  # 4-byte aligned only
    # gating: null / misaligned / bad k
    assert L.moe_topk_gating(None, 4, 8, 2, 1, good, good, None) == -1
    assert L.moe_topk_gating(odd, 4, 8, 2, 1, good, good, None) == -1
    assert L.moe_topk_gating(good, 4, 8, 9, 1, good, good, None) == -1
    assert L.moe_topk_gating(good, 4, 8, 2, 2, good, good, None) == -1
    assert L.moe_topk_gating(good, 0, 8, 2, 1, good, good, None) == 0  # T = 0: nothing enqueued
    # align sort: pointers, then the workspace (missing, misaligned, small)
    aws = moe.moe_align_sort_workspace_bytes(4, 2, 8)
    wsa = _fake(0x300000)
    assert L.moe_align_sort(good, 4, 2, 8, None, good, good, None, wsa, aws, None) == -1
    assert L.moe_align_sort(good, 4, 2, 8, good, good, odd, None, wsa, aws, None) == -1
    assert L.moe_align_sort(good, 4, 2, 8, good, good, good, None, None, aws, None) == -3
    assert L.moe_align_sort(good, 4, 2, 8, good, good, good, None, _fake(0x300010), aws,
                            None) == -3
    assert L.moe_align_sort(good, 4, 2, 8, good, good, good, None, wsa, aws - 1, None) == -3
    assert L.moe_align_sort(good, 0, 2, 8, good, good, good, None, None, 0, None) == 0
    s = moe.make_shape(4, 256, 8, 2, 256, 2)
    S = ctypes.byref(s)
    need = moe.moe_workspace_bytes(s)
    ws = _fake(0x200000)
    # FP8 needs scales
    assert L.moe_grouped_gemm_w13_swiglu(S, good, good, None, good, good, good, good, ws, need,
                                         None) == -1
    # workspace too small / misaligned
    assert L.moe_grouped_gemm_w13_swiglu(S, good, good, good, good, good, good, good, ws, need - 1,
                                         None) == -3
    assert L.moe_grouped_gemm_w13_swiglu(S, good, good, good, good, good, good, good,
                                         _fake(0x200010), need, None) == -3
    assert L.moe_grouped_gemm_w2(S, good, good, None, good, good, good, ws, need, None) == -1
    assert L.moe_combine(S, good, good, None, good, None) == -1
    assert L.moe_fused_forward(S, good, good, good, good, good, None, good, None, None, ws, need,
                               None) == -1
    s2 = moe.make_shape(4, 200, 8, 2, 256, 1)
    assert L.moe_fused_forward(ctypes.byref(s2), good, good, good, None, good, None, good, None,
                               None, ws, 1 << 30, None) == -2
    s0 = moe.make_shape(0, 256, 8, 2, 256, 2)
    assert L.moe_fused_forward(ctypes.byref(s0), good, good, good, good, good, good, good, None,
                               None, ws, moe.moe_workspace_bytes(s0), None) == 0


def test_noalloc_rejects_shapes_beyond_its_scratch(L):
    # the prefill layer needs about 1.2 GB of scratch: refused before any
    # pointer is looked at or anything is enqueued
    s = moe.make_shape(4096, 7168, 256, 8, 2048, 2)
    assert moe.moe_workspace_bytes(s) > moe.NOALLOC_SCRATCH_BYTES
    assert L.moe_fused_forward_noalloc(ctypes.byref(s), None, None, None, None, None, None, None,
                                       None, None, None) == -5
    assert L.moe_status_string(-5)
    s0 = moe.make_shape(0, 7168, 256, 8, 2048, 2)
    assert L.moe_fused_forward_noalloc(ctypes.byref(s0), None, None, None, None, None, None, None,
                                       None, None, None) == 0
    bad = moe.make_shape(4, 100, 8, 2, 256, 2)
    assert L.moe_fused_forward_noalloc(ctypes.byref(bad), None, None, None, None, None, None,
                                       None, None, None, None) == -2


def test_inv_rope_rejects_before_launch(L):
    good = _fake(0x100000)
    odd = _fake(0x100004)
    f = L.moe_inv_rope_fp8_quant
    assert f(good, good, good, 4, 8, 100, 64, 16, 0, good, good, None) == -2  # head_dim % 16
    assert f(good, good, good, 4, 8, 128, 136, 16, 0, good, good, None) == -2  # rot > head
    assert f(good, good, good, 4, 8, 1024, 128, 16, 0, good, good, None) == -2  # head > 512
    assert f(good, good, good, 4, 8, 128, 0, 16, 0, good, good, None) == -2
    assert f(good, good, good, 4, 0, 128, 128, 16, 0, good, good, None) == -1
    assert f(good, good, good, 4, 8, 128, 128, 0, 0, good, good, None) == -1
    assert f(good, good, good, 4, 8, 128, 128, 16, 2, good, good, None) == -1
    assert f(None, good, good, 4, 8, 128, 128, 16, 0, good, good, None) == -1
    assert f(good, good, good, 4, 8, 128, 128, 16, 0, odd, good, None) == -1
    assert f(good, good, good, -1, 8, 128, 128, 16, 0, good, good, None) == -1
    assert f(None, None, None, 0, 8, 128, 128, 16, 0, None, None, None) == 0  # T = 0


def test_act_quant_rejects_before_launch(L):
    good = _fake(0x100000)
    odd = _fake(0x100004)
    assert L.moe_act_quant_e4m3(None, 64, good, good, None) == -1
    assert L.moe_act_quant_e4m3(good, 64, None, good, None) == -1
    assert L.moe_act_quant_e4m3(good, 64, good, None, None) == -1
    assert L.moe_act_quant_e4m3(odd, 64, good, good, None) == -1
    assert L.moe_act_quant_e4m3(good, 64, good, odd, None) == -1
    assert L.moe_act_quant_e4m3(good, 12, good, good, None) == -1  # not a multiple of 8
    assert L.moe_act_quant_e4m3(good, -8, good, good, None) == -1
    assert L.moe_act_quant_e4m3(good, 0, good, good, None) == 0  # nothing enqueued


def test_router_entry_points_reject_before_launch(L):
    good = _fake(0x100000)
    odd = _fake(0x100004)
    s = moe.make_shape(4, 256, 8, 2, 256, 2)
    S = ctypes.byref(s)
    need = moe.moe_workspace_bytes(s)
    ws = _fake(0x200000)
    assert L.moe_router_logits(S, None, good, good, ws, need, None) == -1
    assert L.moe_router_logits(S, good, odd, good, ws, need, None) == -1
    assert L.moe_router_logits(S, good, good, None, ws, need, None) == -1
    assert L.moe_router_logits(S, good, good, good, ws, need - 1, None) == -3
    s0 = moe.make_shape(0, 256, 8, 2, 256, 2)
    assert L.moe_router_logits(ctypes.byref(s0), good, good, good, ws, need, None) == 0
    # the layer's arguments are checked before the router is enqueued: FP8
    # without scales, a misaligned output, a null router matrix
    assert L.moe_fused_forward_router(S, good, good, good, None, good, good, good, None, None,
                                      None, ws, need, None) == -1
    assert L.moe_fused_forward_router(S, good, good, good, good, good, good, odd, None, None,
                                      None, ws, need, None) == -1
    assert L.moe_fused_forward_router(S, good, None, good, good, good, good, good, None, None,
                                      None, ws, need, None) == -1
    assert L.moe_fused_forward_router(ctypes.byref(s0), good, good, good, good, good, good, good,
                                      None, None, None, ws, need, None) == 0


def test_missing_library_fails_loudly(monkeypatch):
    # the product path has no fallback: without the HIP library every entry
    # point raises instead of computing anything elsewhere
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libmoe_gfx950.so"))
    with pytest.raises(moe.MoeError):
        moe.lib()
    with pytest.raises(moe.MoeError):
        moe.moe_workspace_bytes(moe.make_shape(4, 256, 8, 2, 256, 2))


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
