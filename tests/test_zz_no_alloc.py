"""moe_fused_forward_noalloc, the entry point for callers that cannot
allocate, against moe_fused_forward through the C ABI: the same kernels run
on the library's static scratch instead of a caller workspace, so outputs,
ids and weights must be bit-identical, and the output within the per-mode
tolerance of the CPU oracle.  Two calls in a row share the scratch; the
second has a smaller input, so stale values of the first call must not leak
into it."""
import numpy as np
import pytest
import torch

import moe_layer_gating_amd as moe
import moe_workloads as wl
import oracle
from gpu_helpers import FP8, BF16, OUT_TOL, act_to_numpy, rel_inf, say, upload

pytestmark = pytest.mark.gpu

SHAPES = [
    # name, T, H, E, k, I, mode: few-token (one-block front, swap-AB GEMMs)
    # and many-token (chunked grouping, tiled GEMMs) layers that fit
    ("noalloc_decode_fp8", 16, 512, 64, 8, 256, FP8),
    ("noalloc_tiles_bf16", 1100, 256, 16, 8, 256, BF16),
]


def _run(D, k, mode, T, noalloc):
    H = D["x"].shape[1]
    out = torch.full((T, H), float("nan"), dtype=moe.act_dtype(mode), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    x, lg = D["x"][:T].contiguous(), D["logits"][:T].contiguous()
    if noalloc:
        moe.moe_fused_forward_noalloc(x, lg, D["w13"], D["w13_scale"], D["w2"], D["w2_scale"], k,
                                      out, topk_ids=ids, topk_weights=w)
    else:
        moe.moe_fused_forward(x, lg, D["w13"], D["w13_scale"], D["w2"], D["w2_scale"], k, out=out,
                              topk_ids=ids, topk_weights=w)
    torch.cuda.synchronize()
    return out, ids, w


@pytest.mark.parametrize("c", SHAPES, ids=[c[0] for c in SHAPES])
def test_noalloc_matches_fused_two_calls(c):
    name, T, H, E, k, I, mode = c
    assert torch.cuda.is_available()
    L = wl.make_layer(wl.scaled(name, T, H, E, k, I, mode, routing="zipf", seed=5))
    shape = moe.make_shape(T, H, E, k, I, mode)
    assert moe.moe_workspace_bytes(shape) <= moe.NOALLOC_SCRATCH_BYTES
    D = upload(L)
    for Tc in (T, max(1, T // 3)):  # the second call is smaller
        say("noalloc", name, "T =", Tc)
        o1, i1, w1 = _run(D, k, mode, Tc, noalloc=True)
        o0, i0, w0 = _run(D, k, mode, Tc, noalloc=False)
        assert torch.equal(i1, i0)
        assert torch.equal(w1, w0)
        assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
        ref = oracle.forward(mode, L["x"][:Tc], L["logits"][:Tc], L["w13"], L["w13_scale"],
                             L["w2"], L["w2_scale"], k)
        assert np.array_equal(i1.cpu().numpy(), ref["topk_ids"])
        og = oracle.to_f64(act_to_numpy(o1, mode), mode)
        assert not np.isnan(og).any()
        err = rel_inf(og, ref["out_exact"])
        say("  rel err", err)
        assert err <= OUT_TOL[mode]
