"""GPU parity of the router GEMM and of the layer run from the router
weights (moe_router_logits, moe_fused_forward_router), through the C ABI.

logits: |gpu - ref| <= (H/16 + 64) * 2^-24 * sum_h |x w| elementwise, ref the
oracle's exactly summed logits.  The products are exact on both sides (bf16 x
bf16, or fp32 FMAs); the GPU sums in fp32 in chains of at most H/16 + 64
additions (per-lane FMA chains and a 64-lane tree, or chained MFMAs of 32
products each), each adding at most one rounding of 2^-24 of the running sum
of magnitudes.

The layer: the top-k decision is taken on the logits the GPU produced, so
gating, grouping and the output are checked against the oracle run on those
same logits (ids bit-exact, out within the per-mode tolerance).  Against the
oracle's own exact logits the ids may differ only where two logits of the
token lie within twice the bound above (a near tie); the seeded cases have
none, and the test asserts both.
"""
import numpy as np
import pytest
import torch

import moe_layer_gating_amd as moe
import moe_workloads as wl
import oracle
from gpu_helpers import (BF16, F32, FP8, OUT_TOL, act_to_numpy, act_to_torch, assert_grouping,
                         rel_inf, say, upload)

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()


def _bound(x, wg, mode, H):
    xa = np.abs(oracle.to_f64(x, mode))
    wa = np.abs(oracle.to_f64(wg, mode))
    return (H / 16 + 64) * U * (xa @ wa.T)


ROUTER = [
    # name, T, H, E, mode   (few-token wave kernel unless E % 128 == 0 and T >= 256)
    ("f32_tiny", 16, 128, 8, F32),
    ("bf16_decode", 8, 4096, 8, BF16),
    ("bf16_t1_e64", 1, 4096, 64, BF16),
    ("bf16_t37_ragged_group", 37, 1024, 64, BF16),
    ("bf16_tiles_e128", 512, 768, 128, BF16),
    ("bf16_tiles_e256_ragged", 300, 1024, 256, BF16),
    ("bf16_e96_many_tokens", 260, 512, 96, BF16),
]


@pytest.mark.parametrize("c", ROUTER, ids=[c[0] for c in ROUTER])
def test_router_logits(c):
    name, T, H, E, mode = c
    L = wl.make_layer(wl.scaled(name, T, H, E, 1, 128, mode, seed=len(name)), with_weights=False)
    x, wg = L["x"], L["wg"]
    say("router", name)
    lg = moe.moe_router_logits(act_to_torch(x, mode), act_to_torch(wg, mode))
    torch.cuda.synchronize()
    g = lg.cpu().numpy()
    ref = oracle.router_logits(mode, x, wg)
    d = np.abs(g.astype(np.float64) - ref)
    b = _bound(x, wg, mode, H)
    say("  max err / bound %.3g, median rel err %.3g" % (np.max(d / b), np.median(d / np.abs(ref))))
    assert np.all(d <= b)
    assert np.median(d / np.maximum(np.abs(ref), 1e-30)) < 1e-6


def test_router_zero_tokens_is_noop():
    wg = torch.zeros((8, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 8), 5.0, device="cuda")
    moe.moe_router_logits(torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda"), wg,
                          logits=out[:0])
    torch.cuda.synchronize()
    assert torch.all(out == 5.0)


LAYERS = [
    # name, T, H, E, k, I, mode, routing
    # router computed inside the one-block front kernel (bf16 layers, T*k <=
    # 256, T*E <= 4096, E*H <= 131072): at the limits, ragged expert and
    # token tiles, K split over fewer ranges than waves, and whole 4-tile
    # items per wave (E = 1024)
    ("bf16_decode_router", 8, 1024, 8, 2, 512, BF16, "uniform"),
    ("fp8_decode_router", 16, 1024, 64, 8, 256, FP8, "uniform"),
    ("fp8_front_router_max_te", 32, 1024, 128, 8, 256, FP8, "uniform"),
    ("bf16_front_router_e1024", 4, 128, 1024, 16, 128, BF16, "uniform"),
    ("bf16_front_router_ragged", 3, 384, 33, 5, 128, BF16, "uniform"),
    # separate router kernel: fp32, T*E or E*H just past the front's limits,
    # many pairs
    ("f32_tiny_router", 16, 128, 8, 2, 256, F32, "uniform"),
    ("fp8_router_past_te", 33, 256, 128, 4, 128, FP8, "uniform"),
    ("fp8_router_past_eh", 1, 4096, 64, 8, 256, FP8, "uniform"),
    ("fp8_mixed_router", 512, 768, 128, 8, 256, FP8, "uniform"),
    ("fp8_prefill_router", 600, 512, 256, 8, 256, FP8, "uniform"),
]


@pytest.mark.parametrize("c", LAYERS, ids=[c[0] for c in LAYERS])
def test_fused_forward_router(c):
    name, T, H, E, k, I, mode, routing = c
    L = wl.make_layer(wl.scaled(name, T, H, E, k, I, mode, routing=routing, seed=len(name)))
    D = upload(L)
    wg = act_to_torch(L["wg"], mode)
    lg = torch.full((T, E), float("nan"), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    say("fused router", name)
    shape = moe.make_shape(T, H, E, k, I, mode)
    ws = moe.workspace(shape)
    out = moe.moe_fused_forward_router(D["x"], wg, D["w13"], D["w13_scale"], D["w2"],
                                       D["w2_scale"], k, logits=lg, topk_ids=ids, topk_weights=w,
                                       ws=ws)
    torch.cuda.synchronize()
    views = moe.routing_from_workspace(ws, T, E, k)
    grp = {n: views[n].cpu().numpy().copy() for n in ("counts", "offsets", "sorted_ids",
                                                      "inv_perm")}
    g = lg.cpu().numpy()
    exact = oracle.router_logits(mode, L["x"], L["wg"])
    b = _bound(L["x"], L["wg"], mode, H)
    assert np.all(np.abs(g.astype(np.float64) - exact) <= b)
    # the layer on the GPU's own logits
    ref = oracle.forward(mode, L["x"], g, L["w13"], L["w13_scale"], L["w2"], L["w2_scale"], k)
    assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert np.max(np.abs(w.cpu().numpy() - ref["topk_weights"])) <= 1e-6
    assert_grouping(grp, ref["counts"], ref["offsets"], ref["sorted_ids"], ref["inv_perm"])
    # without the logits output the call computes the same layer
    ids2 = torch.empty((T, k), dtype=torch.int32, device="cuda")
    out2 = moe.moe_fused_forward_router(D["x"], wg, D["w13"], D["w13_scale"], D["w2"],
                                        D["w2_scale"], k, topk_ids=ids2)
    torch.cuda.synchronize()
    assert torch.equal(ids2, ids)
    assert torch.equal(out2.view(torch.int16) if mode else out2, out.view(torch.int16) if mode else out)
    og = oracle.to_f64(act_to_numpy(out, mode), mode)
    err = rel_inf(og, ref["out_exact"])
    say("  rel err", err)
    assert err <= OUT_TOL[mode]
    # against the exact logits: any different choice must be a near tie
    rid, _ = oracle.topk_gating(exact, k)
    gid = ids.cpu().numpy()
    diff_rows = np.where(np.any(rid != gid, axis=1))[0]
    for t in diff_rows:
        srt = np.sort(exact[t])[::-1]
        gaps = srt[:k] - srt[1:k + 1]
        assert np.min(gaps) <= 2 * np.max(b[t]), "row %d differs without a near tie" % t
    say("  rows choosing differently from the exact logits:", len(diff_rows))
    assert len(diff_rows) == 0
