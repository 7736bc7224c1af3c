"""The fused entry points captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay, with eager work and synchronisations between the
replays, must reproduce the eagerly launched result bit for bit.  The layer
enqueues no memset and no host synchronisation, so it is capturable; this
checks that replays after the first stay correct (control words and counters
are re-zeroed by kernels inside the graph)."""
import numpy as np
import pytest
import torch

import moe_layer_gating_amd as moe
import moe_workloads as wl
from gpu_helpers import BF16, FP8, say, upload

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, E, k, I, mode, routing
    ("graph_fp8_decode", 4, 512, 32, 8, 256, FP8, "uniform"),
    ("graph_bf16_decode", 8, 256, 8, 2, 384, BF16, "uniform"),
    ("graph_fp8_tiles", 300, 256, 8, 4, 256, FP8, "zipf"),
    ("graph_fp8_chunked_sort", 1100, 256, 16, 8, 128, FP8, "uniform"),
]


# the router entry point (router GEMM in front): its few-token and tiled paths
ROUTER_CASES = [
    ("graph_router_decode", 4, 512, 32, 8, 256, FP8, "uniform"),
    ("graph_router_tiles", 300, 256, 128, 8, 128, FP8, "uniform"),
]


@pytest.mark.parametrize("c", CASES + ROUTER_CASES, ids=[c[0] for c in CASES + ROUTER_CASES])
def test_graph_replays_match_eager(c):
    assert torch.cuda.is_available()
    name, T, H, E, k, I, mode, routing = c
    L = wl.make_layer(wl.scaled(name, T, H, E, k, I, mode, routing=routing, seed=5))
    D = upload(L)
    shape = moe.make_shape(T, H, E, k, I, mode)
    ws = moe.workspace(shape)
    out = torch.empty((T, H), dtype=moe.act_dtype(mode), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    router = name.startswith("graph_router")
    wg = torch.from_numpy(L["wg"].view(np.int16)).view(torch.bfloat16).cuda() if router else None

    def step():
        if router:
            moe.moe_fused_forward_router(D["x"], wg, D["w13"], D["w13_scale"], D["w2"],
                                         D["w2_scale"], k, out=out, ws=ws, topk_ids=ids)
        else:
            moe.moe_fused_forward(D["x"], D["logits"], D["w13"], D["w13_scale"], D["w2"],
                                  D["w2_scale"], k, out=out, ws=ws, topk_ids=ids)

    say("graph", name)
    step()
    torch.cuda.synchronize()
    want = out.view(torch.int16).cpu().numpy().copy()
    want_ids = ids.cpu().numpy().copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream before capturing
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), want), "replay %d" % rep
        assert np.array_equal(ids.cpu().numpy(), want_ids), "replay %d" % rep
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(out.view(torch.int16).cpu().numpy(), want)
