"""GPU parity of the inverse rotary embedding + per-head FP8 quantisation
(moe_inv_rope_fp8_quant) against the CPU oracle, through the C ABI.

The e4m3 codes and the per-(token, head) scales are integer decisions and
values taken on fp32 numbers that both sides form with the same single fp32
operations, so both are compared bit for bit: every code, every scale.
Shapes: head sizes 16..512, partial rotation, both pairings, one token and
the 4096-token prefill batch, decode positions, zero heads, values across
the bf16 range (saturation and subnormal codes), positions outside the
table (clamped), and T = 0 (nothing written).
"""
import numpy as np
import pytest
import torch

import moe_layer_gating_amd as moe
import moe_workloads as wl
import oracle
from gpu_helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()


def _run(x, pos, cs, inter):
    xt = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    codes = torch.full(x.shape, 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full(x.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_inv_rope_fp8_quant(xt, torch.from_numpy(pos).cuda(), torch.from_numpy(cs).cuda(),
                               interleaved=inter, codes=codes, scales=scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _check(x, pos, cs, inter, name):
    say("inv rope fp8", name, x.shape, "rot", cs.shape[1], "interleaved", inter)
    c, s = _run(x, pos, cs, inter)
    rc, rs, _ = oracle.inv_rope_fp8(x, pos, cs, interleaved=inter)
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), "scales differ"
    assert np.array_equal(c, rc), "codes differ: %d of %d" % (np.sum(c != rc), c.size)


CASES = [
    # name, T, heads, head_dim, rot_dim, max_pos, interleaved, positions
    ("decode_llama", 16, 32, 128, 128, 8192, False, "random"),
    ("one_token", 1, 8, 128, 128, 4096, True, "random"),
    ("partial_rot", 37, 6, 192, 64, 2048, False, "prefill"),
    ("partial_rot_inter", 29, 5, 80, 48, 512, True, "random"),
    ("small_heads", 300, 3, 16, 16, 1024, False, "prefill"),
    ("big_heads", 9, 4, 512, 256, 1024, True, "random"),
    ("head256", 50, 16, 256, 256, 65536, False, "random"),
]


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_inv_rope_fp8(c):
    name, T, nh, hd, rot, maxp, inter, posk = c
    R = wl.make_rope(wl.scaled_rope(name, T, nh, hd, rot, maxp, inter, posk, seed=len(name)))
    _check(R["x"], R["positions"], R["cos_sin"], inter, name)


@pytest.mark.parametrize("name", ["rope_prefill", "rope_decode"])
def test_inv_rope_fp8_workloads(name):
    R = wl.make_rope(wl.ROPE_WORKLOADS[name])
    _check(R["x"], R["positions"], R["cos_sin"], R["spec"].interleaved, name)


@pytest.mark.parametrize("inter", [False, True])
def test_inv_rope_fp8_value_range(inter):
    """bf16 values from every binade (heads whose magnitudes spread over many
    binades: subnormal codes, saturation at +-448), zero heads, one huge
    element per head, and positions outside the table."""
    rng = np.random.default_rng(5)
    T, nh, hd, rot, maxp = 64, 8, 128, 96, 300
    e = rng.integers(1, 254, (T, nh, hd)).astype(np.uint16)
    m = rng.integers(0, 128, (T, nh, hd)).astype(np.uint16)
    sgn = (rng.random((T, nh, hd)) < 0.5).astype(np.uint16) << 15
    x = (sgn | (e << 7) | m).astype(np.uint16)
    # narrow heads: magnitudes within a few binades of each other
    for t in range(0, T, 4):
        x[t] = ((x[t] & 0x807F) | ((100 + rng.integers(0, 6, (nh, hd))) << 7)).astype(np.uint16)
    x[3, :, :] = 0
    x[5, 2, :] = 0x8000  # -0 only
    x[7, :, 0] = 0x7F7F  # the largest finite bf16
    pos = rng.integers(-50, maxp + 50, T).astype(np.int32)
    cs = wl.rope_table(maxp, rot)
    _check(x, pos, cs, inter, "value range")


def test_inv_rope_fp8_zero_tokens():
    x = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    codes = torch.full((1, 4, 64), 7, dtype=torch.uint8, device="cuda")
    scales = torch.full((1, 4), 3.0, device="cuda")
    moe.moe_inv_rope_fp8_quant(x, torch.zeros(0, dtype=torch.int32, device="cuda"),
                               torch.ones((8, 64), device="cuda"), codes=codes[:0],
                               scales=scales[:0])
    torch.cuda.synchronize()
    assert torch.all(codes == 7) and torch.all(scales == 3.0)
