"""GPU parity of every step of the fused MoE layer against the CPU oracle,
called through the C ABI (via the ctypes binding), on seeded layers small
enough for the oracle to finish in seconds.  The shapes span several GEMM
tiles, ragged tails (experts with token counts that are not multiples of the
16-wide tile), skewed and empty experts, T = 1, k = 1, E = 1 and k = E.

Bars: routing (ids, counts, offsets, sorted ids, inverse permutation) and
the FP8 activation scales are bit-exact; the layer output is within the
per-mode tolerance on max|gpu - ref| / max|ref| (fp32 1e-5, bf16 5e-3, FP8
2e-2), ref being the oracle's output before its final rounding to the
output type (both sides rounding to bf16 could otherwise differ by one
output ulp, up to 2^-7 of max|ref|, for results that are both correct).
Stage bars are tighter: h within one bf16 step of the oracle (see
gpu_helpers.bf16_step_ratio) and at least 99% of its bf16 values identical,
95% in the tiled FP8 kernels, whose gate/up products go through the FP8
MFMA (gpu_helpers.h_identical_min); y (fp32) within 1e-5, except FP8 where
the down projection's FP8 MFMA rounds its sums (about 2^-19 of sum|p| per
instruction, measured) and the bar is 2e-4.
Each stage is fed the oracle's upstream outputs so a failure names its stage.
"""
import numpy as np
import pytest
import torch

import moe_layer_gating_amd as moe
import moe_workloads as wl
import oracle
from gpu_helpers import (BF16, F32, FP8, OUT_TOL, act_to_numpy, act_to_torch, assert_grouping,
                         bf16_step_ratio, f32_tensor, fused_call, h_identical_min, int_tensor,
                         rel_inf, say, upload)

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, E, k, I, mode, routing
    ("f32_tiny_layer", 16, 128, 8, 2, 256, F32, "uniform"),
    ("f32_ragged", 37, 256, 6, 3, 384, F32, "uniform"),
    ("f32_single_expert", 5, 128, 1, 1, 128, F32, "uniform"),
    ("bf16_small", 11, 512, 8, 2, 384, BF16, "uniform"),
    ("bf16_multitile", 70, 256, 4, 2, 256, BF16, "uniform"),
    ("bf16_k1", 9, 256, 4, 1, 128, BF16, "uniform"),
    ("fp8_small", 16, 512, 16, 4, 256, FP8, "uniform"),
    ("fp8_zipf", 96, 512, 32, 8, 512, FP8, "zipf"),
    ("fp8_empty", 40, 384, 20, 4, 256, FP8, "empty"),
    ("fp8_t1", 1, 512, 64, 8, 256, FP8, "uniform"),
    ("fp8_k_equals_E", 6, 256, 4, 4, 128, FP8, "uniform"),
    # few pairs per expert with more than 256 pairs: the multi-kernel front
    # (gating, grouping and tile-list kernels) instead of the one-block one
    ("fp8_skinny_many_pairs", 40, 256, 64, 8, 256, FP8, "uniform"),
    # few-token class at 48, 96 and 256 pairs (about 40, 65 and 20 tiles)
    ("fp8_skinny_48_pairs", 6, 256, 64, 8, 256, FP8, "uniform"),
    ("bf16_skinny_96_pairs", 12, 256, 128, 8, 256, BF16, "uniform"),
    ("fp8_skinny_256_pairs", 32, 256, 64, 8, 256, FP8, "zipf"),
    ("bf16_skinny_t100", 100, 256, 16, 2, 256, BF16, "uniform"),
    ("bf16_skinny_t200", 200, 256, 32, 2, 128, BF16, "uniform"),
    # many pairs per expert: the 128-position tiled GEMMs (several tiles per
    # expert, ragged last tiles, 8+ weight-row blocks, empty and skewed experts)
    ("fp8_tiles_ragged", 600, 512, 8, 2, 512, FP8, "uniform"),
    ("bf16_tiles_zipf", 256, 384, 16, 4, 384, BF16, "zipf"),
    ("fp8_tiles_empty", 256, 256, 16, 4, 640, FP8, "empty"),
    ("bf16_tiles_one_expert", 200, 256, 1, 1, 512, BF16, "uniform"),
    # two experts with runs of dozens of 128-position tiles each (a skewed
    # split, ragged last tiles, more tiles than one row block's XCD share)
    ("fp8_tiles_long_runs", 9300, 128, 2, 1, 128, FP8, "zipf"),
    # 256 or more pairs per expert: many full 128-position tiles per expert,
    # heavy skew, ragged last tiles of every width
    ("fp8_tiles_heavy_zipf", 3000, 256, 8, 2, 256, FP8, "zipf"),
    ("bf16_tiles_heavy", 2900, 256, 8, 1, 384, BF16, "uniform"),
    ("fp8_tiles_heavy_h384", 1100, 384, 4, 1, 256, FP8, "uniform"),
    # 128-position tiles whose rows are one 128-byte K stage long (H = I =
    # 128 in FP8): every prefetch index is clamped to that stage
    ("fp8_tiles128_one_stage", 600, 128, 4, 2, 128, FP8, "uniform"),
    # 16 <= mean pairs per expert < 64: 64-position tiles, some experts spill
    # into a second tile
    ("fp8_tiles64_ragged", 250, 384, 8, 2, 384, FP8, "uniform"),
    # 8192 pairs or more: the grouping runs as a chunked counting sort (ragged
    # last chunk) inside the fused entry point
    ("fp8_tiles_chunked_sort", 1100, 256, 16, 8, 256, FP8, "zipf"),
    # chunked grouping with 128-position tiles and under 256 pairs per
    # expert: the down projection takes the spread tile order (full tiles
    # evenly among the partial ones of the skewed experts)
    ("fp8_tiles_spread_zipf", 1200, 256, 64, 8, 256, FP8, "zipf"),
    ("bf16_tiles_chunked_sort", 4200, 128, 64, 2, 128, BF16, "uniform"),
    # the interface's largest expert count and top-k (E = 1024, k = 16): 256
    # pairs, the most the one-block front kernel takes; 272 pairs, just past
    # it; and 16 pairs per expert on average, the smallest mean that takes the
    # tiled GEMMs, with the chunked grouping over all 1024 experts
    ("bf16_max_E_k", 16, 128, 1024, 16, 128, BF16, "uniform"),
    ("fp8_max_E_k_multi", 17, 128, 1024, 16, 128, FP8, "uniform"),
    # one-block front with an x too large for its quantising block (T*H >
    # 131072): x goes to the grid-wide amax and quantisation passes
    ("fp8_front_big_x", 64, 4096, 64, 4, 128, FP8, "uniform"),
    ("fp8_tiles_max_E", 1024, 128, 1024, 16, 128, FP8, "uniform"),
]
IDS = [c[0] for c in CASES]

_cache = {}


def case(c):
    if c[0] not in _cache:
        name, T, H, E, k, I, mode, routing = c
        L = wl.make_layer(wl.scaled(name, T, H, E, k, I, mode, routing=routing, seed=len(name)))
        ref = oracle.forward(mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"],
                             L["w2_scale"], k)
        _cache[c[0]] = (L, ref)
    return _cache[c[0]]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_gating(c):
    L, ref = case(c)
    k = c[4]
    say("gating", c[0])
    ids, w = moe.moe_topk_gating(torch.from_numpy(L["logits"]).cuda(), k)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert np.max(np.abs(w.cpu().numpy() - ref["topk_weights"])) <= 1e-6


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_align_sort(c):
    L, ref = case(c)
    E = c[3]
    say("align_sort", c[0])
    counts, offsets, sorted_ids, inv = moe.moe_align_sort(int_tensor(ref["topk_ids"]), E)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(sorted_ids.cpu().numpy(), ref["sorted_ids"])
    assert np.array_equal(inv.cpu().numpy(), ref["inv_perm"])


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_w13_swiglu(c):
    L, ref = case(c)
    mode, k = c[6], c[4]
    D = upload(L)
    say("w13", c[0])
    h, sc = moe.moe_grouped_gemm_w13_swiglu(D["x"], D["w13"], D["w13_scale"],
                                            int_tensor(ref["sorted_ids"]), int_tensor(ref["offsets"]),
                                            k)
    torch.cuda.synchronize()
    hg = act_to_numpy(h, mode)
    hv, rv = oracle.to_f64(hg, mode), oracle.to_f64(ref["h"], mode)
    if mode == F32:
        assert rel_inf(hv, rv) <= 1e-5
    else:
        # every element within one bf16 step of the oracle's (see
        # bf16_step_ratio), almost all equal
        assert bf16_step_ratio(hv, rv) <= 1.0
        assert np.mean(hg == ref["h"]) >= h_identical_min(mode, c[1], k, c[3])
    if mode == FP8:
        s = sc.cpu().numpy()
        _, s_x, _ = oracle.act_quant(L["x"], BF16)
        assert s[0] == s_x  # bit-exact activation scale
        assert s[2] == np.float32(np.max(np.abs(oracle.to_f64(L["x"], BF16))))
        assert s[3] == np.float32(np.max(np.abs(hv)))  # amax(h) of the GPU's own h
        assert s[1] == np.float32(s[3]) / np.float32(448.0)


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_w2(c):
    L, ref = case(c)
    mode, k = c[6], c[4]
    D = upload(L)
    # inputs: the oracle's h and, in FP8 mode, the oracle's scale of it
    act = np.zeros(4, np.float32)
    if mode == FP8:
        _, s_h, _ = oracle.act_quant(ref["h"], BF16)
        act[1] = s_h
        act[3] = np.float32(np.max(np.abs(oracle.to_f64(ref["h"], BF16))))
    say("w2", c[0])
    y = moe.moe_grouped_gemm_w2(act_to_torch(ref["h"], mode), D["w2"], D["w2_scale"],
                                int_tensor(ref["offsets"]), f32_tensor(act), k)
    torch.cuda.synchronize()
    y_ref, _ = oracle.w2(mode, ref["h"], L["w2"], L["w2_scale"], ref["offsets"], k)
    assert rel_inf(y.cpu().numpy(), y_ref) <= (2e-4 if mode == FP8 else 1e-5)


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_combine(c):
    L, ref = case(c)
    mode, k, E = c[6], c[4], c[3]
    y_ref, _ = oracle.w2(mode, ref["h"], L["w2"], L["w2_scale"], ref["offsets"], k)
    y32 = y_ref.astype(np.float32)
    say("combine", c[0])
    out = moe.moe_combine(f32_tensor(y32), int_tensor(ref["inv_perm"]),
                          f32_tensor(ref["topk_weights"]), mode, E=E)
    torch.cuda.synchronize()
    want = oracle.combine(mode, y32, ref["inv_perm"], ref["topk_weights"])
    og = act_to_numpy(out, mode)
    if mode == F32:
        assert rel_inf(og, want) <= 1e-6
    else:
        assert rel_inf(oracle.to_f64(og, mode), oracle.to_f64(want, mode)) <= 4e-3
        assert np.mean(og == want) > 0.99


@pytest.mark.parametrize("c", CASES, ids=IDS)
def test_fused_forward(c):
    L, ref = case(c)
    mode, k = c[6], c[4]
    D = upload(L)
    T, H = c[1], c[2]
    out = torch.full((T, H), float("nan"), dtype=moe.act_dtype(mode), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    say("fused", c[0])
    _, grp = fused_call(D, k, mode, out=out, topk_ids=ids, topk_weights=w)
    assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert np.max(np.abs(w.cpu().numpy() - ref["topk_weights"])) <= 1e-6
    # the grouping this call's own kernels wrote (one-block front, one block
    # per expert, or the chunked sort, by pair count)
    assert_grouping(grp, ref["counts"], ref["offsets"], ref["sorted_ids"], ref["inv_perm"])
    og = oracle.to_f64(act_to_numpy(out, mode), mode)
    assert not np.isnan(og).any()  # every row written
    # reference: the oracle's output before its rounding to the output type
    err = rel_inf(og, ref["out_exact"])
    say("  rel err", err)
    assert err <= OUT_TOL[mode]
    # a second call gives bit-identical results
    out2 = moe.moe_fused_forward(D["x"], D["logits"], D["w13"], D["w13_scale"], D["w2"],
                                 D["w2_scale"], k)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if mode else out, out2.view(torch.int16) if mode else out2)


def test_fused_zero_input_fp8():
    L, ref = case(CASES[6])
    D = upload(L)
    x = torch.zeros_like(D["x"])
    say("fused zero x")
    out = moe.moe_fused_forward(x, D["logits"], D["w13"], D["w13_scale"], D["w2"], D["w2_scale"], 4)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out.float()).item() == 0


def test_fused_t0_is_noop():
    L, ref = case(CASES[0])
    D = upload(L)
    out = torch.full((1, 128), 7.0, device="cuda")
    say("fused T=0")
    moe.moe_fused_forward(D["x"][:0], D["logits"][:0], D["w13"], None, D["w2"], None, 2, out=out[:0])
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_gating_ties_and_neginf():
    rng = np.random.default_rng(7)
    for kind in range(3):
        T, E, k = 50, 64, 8
        if kind == 0:
            l = rng.integers(-2, 3, (T, E)).astype(np.float32)
        elif kind == 1:
            l = rng.standard_normal((T, E)).astype(np.float32)
            l[:, ::3] = -np.inf
        else:
            l = rng.choice(np.array([0.0, -0.0, -1.0], np.float32), (T, E)).astype(np.float32)
        say("gating adversarial", kind)
        for renorm in (True, False):
            ids, w = moe.moe_topk_gating(torch.from_numpy(l).cuda(), k, renorm)
            torch.cuda.synchronize()
            rid, rw = oracle.topk_gating(l, k, renorm)
            assert np.array_equal(ids.cpu().numpy(), rid)
            assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6


@pytest.mark.parametrize("E,k,T", [(64, 8, 32), (128, 8, 16), (100, 6, 20), (5, 5, 3), (8, 2, 16)])
def test_fused_front_gating_ties_and_neginf(E, k, T):
    """The fused entry point's one-block front kernel (T*k <= 256) selects by
    ranks for E <= 128: ids bit-exact and weights within 1e-6 of the oracle on
    tie-heavy, -inf and signed-zero logits, with both weight rules; the
    grouping the same kernel writes into the workspace (counts, offsets,
    sorted ids, inverse permutation) is bit-exact against the oracle's
    grouping of those ids."""
    rng = np.random.default_rng(E * 100 + k)
    L = wl.make_layer(wl.scaled("front_%d_%d" % (E, k), T, 128, E, k, 128, BF16, seed=E + k))
    D = upload(L)
    for kind in range(3):
        if kind == 0:
            l = rng.integers(-2, 3, (T, E)).astype(np.float32)
        elif kind == 1:
            l = rng.standard_normal((T, E)).astype(np.float32)
            if E - len(range(1, E, 3)) >= k:  # keep >= k finite entries per row
                l[:, 1::3] = -np.inf
        else:
            l = rng.choice(np.array([0.0, -0.0, -1.0], np.float32), (T, E)).astype(np.float32)
        for renorm in (True, False):
            say("fused front gating E=%d k=%d kind=%d renorm=%d" % (E, k, kind, renorm))
            ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
            w = torch.empty((T, k), dtype=torch.float32, device="cuda")
            Dl = dict(D, logits=torch.from_numpy(l).cuda())
            _, grp = fused_call(Dl, k, BF16, renormalize=renorm, topk_ids=ids, topk_weights=w)
            rid, rw = oracle.topk_gating(l, k, renorm)
            assert np.array_equal(ids.cpu().numpy(), rid)
            assert np.max(np.abs(w.cpu().numpy() - rw)) <= 1e-6
            assert_grouping(grp, *oracle.align_sort(rid, E))


def _act_quant_case(bits):
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    codes, sc = moe.moe_act_quant_e4m3(x)
    torch.cuda.synchronize()
    rc, rs, _ = oracle.act_quant(bits, BF16)
    assert np.array_equal(codes.cpu().numpy(), rc)
    got = sc.cpu().numpy()
    assert got[0] == rs  # bit-exact scale
    assert got[1] == np.float32(np.max(np.abs(oracle.to_f64(bits, BF16))))


def test_act_quant_every_finite_bf16():
    """The per-tensor e4m3 quantisation step (x before the gate/up
    projection, h before the down projection): codes and scale bit-exact
    against the oracle's codec, over every finite bf16 value (amax 2^128 -
    2^120 makes the smallest values subnormal or zero codes), then over the
    same values rescaled so that every bf16 binade lands on the codes."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = allb[(allb & 0x7F80) != 0x7F80]
    bits = np.concatenate([finite, np.zeros((-finite.size) % 8, np.uint16)])
    say("act quant: %d finite bf16 values" % finite.size)
    _act_quant_case(bits)
    # the values of exponent field e (|v| in [2^(e-127), 2^(e-126))) with
    # amax set by a single 2^(e-127+8) entry: codes over the whole range
    for e in (1, 60, 120, 127, 140, 200, 246):
        man = np.arange(256, dtype=np.uint16)
        vals = np.concatenate([(e << 7) | (man & 0x7F), 0x8000 | (e << 7) | (man & 0x7F)])
        top = np.array([min(e + 8, 254) << 7], np.uint16)
        b = np.concatenate([vals, top, np.zeros(7, np.uint16)]).astype(np.uint16)
        _act_quant_case(b)


def test_act_quant_zero_and_random():
    _act_quant_case(np.zeros(64, np.uint16))  # amax 0: scale 1, codes 0
    rng = np.random.default_rng(9)
    for sigma in (1e-3, 1.0, 300.0):
        v = (rng.standard_normal(4096 * 8) * sigma).astype(np.float32)
        bits = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        _act_quant_case(bits)


def test_align_sort_large_skewed():
    rng = np.random.default_rng(8)
    T, k, E = 4096, 8, 256
    # Zipf-like ids: many pairs on a few experts, several experts empty
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    say("align_sort large")
    counts, offsets, sorted_ids, inv = moe.moe_align_sort(int_tensor(ids), E)
    torch.cuda.synchronize()
    rc, ro, rs, ri = oracle.align_sort(ids, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(sorted_ids.cpu().numpy(), rs)
    assert np.array_equal(inv.cpu().numpy(), ri)


@pytest.mark.parametrize("T,k,E", [(32, 8, 64), (128, 2, 1024), (257, 1, 8), (300, 8, 64),
                                   (1023, 8, 256), (1024, 8, 256), (4097, 2, 1024),
                                   (700, 16, 33)])
def test_align_sort_every_grouping_kernel(T, k, E):
    """moe_align_sort at and around the pair counts where the grouping kernel
    changes (256 pairs: one block; below 8192: one block per expert; 8192
    and more: the chunked counting sort), with uniform and Zipf-skewed ids;
    every output bit-exact, and inv_perm may be omitted."""
    rng = np.random.default_rng(T * 31 + E)
    for skew in (False, True):
        p = 1.0 / np.arange(1, E + 1) ** 1.1 if skew else np.ones(E)
        p = p / p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)])
        ids = ids.astype(np.int32)
        say("align_sort T=%d k=%d E=%d skew=%d (%d pairs)" % (T, k, E, skew, T * k))
        counts, offsets, sorted_ids, inv = moe.moe_align_sort(int_tensor(ids), E)
        c2, o2, s2, _ = moe.moe_align_sort(int_tensor(ids), E, with_inv=False)
        torch.cuda.synchronize()
        rc, ro, rs, ri = oracle.align_sort(ids, E)
        got = dict(counts=counts.cpu().numpy(), offsets=offsets.cpu().numpy(),
                   sorted_ids=sorted_ids.cpu().numpy(), inv_perm=inv.cpu().numpy())
        assert_grouping(got, rc, ro, rs, ri)
        assert np.array_equal(c2.cpu().numpy(), rc) and np.array_equal(o2.cpu().numpy(), ro)
        assert np.array_equal(s2.cpu().numpy(), rs)


def test_gating_nan_logits_stay_in_range():
    """NaN logits break the contract; both gating kernels read them as -inf,
    so the ids stay inside [0, E) (and equal the oracle's ids on the logits
    with NaN replaced by -inf) and the fused call's grouping stays in range."""
    rng = np.random.default_rng(11)
    T, E, k = 24, 64, 8
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[rng.random((T, E)) < 0.3] = np.nan
    l[3, :] = np.nan  # a row of NaN only
    l[4, : E - 2] = np.nan  # fewer than k non-NaN entries
    clean = np.where(np.isnan(l), np.float32(-np.inf), l)
    rid, _ = oracle.topk_gating(clean, k)
    say("gating NaN logits")
    ids, _ = moe.moe_topk_gating(torch.from_numpy(l).cuda(), k)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), rid)
    L = wl.make_layer(wl.scaled("nan_front", T, 128, E, k, 128, BF16, seed=3))
    D = dict(upload(L), logits=torch.from_numpy(l).cuda())
    ids2 = torch.empty((T, k), dtype=torch.int32, device="cuda")
    _, grp = fused_call(D, k, BF16, topk_ids=ids2)
    assert np.array_equal(ids2.cpu().numpy(), rid)
    assert_grouping(grp, *oracle.align_sort(rid, E))


# Planted routing: expert counts on both sides of the tile boundaries and of
# the quarter / half / full main-loop widths (0, 1, 15-17, 31-33, 63-65, 96,
# 127-129, 255-257, 540, ...), so experts get exact, ragged and single-row
# last tiles.  The last layer has 8400
# pairs: grouping by the chunked counting sort.
PLANTED = [
    # name, T, H, E, k, I, mode, counts
    ("fp8_planted_tile_edges", 1726, 256, 13, 1, 256, FP8,
     [0, 1, 127, 128, 129, 255, 256, 540, 32, 33, 64, 65, 96]),
    ("bf16_planted_tile_edges", 1726, 384, 13, 1, 128, BF16,
     [96, 65, 64, 33, 32, 540, 256, 255, 129, 128, 127, 1, 0]),
    ("fp8_planted_tiles64", 700, 256, 16, 1, 256, FP8,
     [0, 1, 15, 16, 17, 63, 64, 65, 100, 127, 128, 33, 32, 31, 8, 0]),
    ("fp8_planted_chunked", 4200, 256, 8, 2, 128, FP8, [0, 256, 257, 511, 1024, 1280, 2520, 2552]),
]


@pytest.mark.parametrize("c", PLANTED, ids=[c[0] for c in PLANTED])
def test_planted_tile_edges(c):
    name, T, H, E, k, I, mode, counts = c
    L = wl.make_layer(wl.scaled(name, T, H, E, k, I, mode, seed=len(name)))
    L["logits"] = wl.planted_logits(T, E, k, counts, seed=len(name))
    ref = oracle.forward(mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"],
                         L["w2_scale"], k)
    assert np.array_equal(ref["counts"], np.array(counts, np.int32))
    D = upload(L)
    say("planted fused", name)
    out, grp = fused_call(D, k, mode)
    assert np.array_equal(grp["topk_ids"], ref["topk_ids"])
    assert_grouping(grp, ref["counts"], ref["offsets"], ref["sorted_ids"], ref["inv_perm"])
    og = oracle.to_f64(act_to_numpy(out, mode), mode)
    assert not np.isnan(og).any()
    err = rel_inf(og, ref["out_exact"])
    say("  rel err", err)
    assert err <= OUT_TOL[mode]
    say("planted steps", name)
    h, sc = moe.moe_grouped_gemm_w13_swiglu(D["x"], D["w13"], D["w13_scale"],
                                            int_tensor(ref["sorted_ids"]), int_tensor(ref["offsets"]),
                                            k)
    torch.cuda.synchronize()
    hg = act_to_numpy(h, mode)
    assert bf16_step_ratio(oracle.to_f64(hg, mode), oracle.to_f64(ref["h"], mode)) <= 1.0
    assert np.mean(hg == ref["h"]) >= h_identical_min(mode, T, k, E)
    act = np.zeros(4, np.float32)
    if mode == FP8:
        _, s_h, _ = oracle.act_quant(ref["h"], BF16)
        act[1] = s_h
        act[3] = np.float32(np.max(np.abs(oracle.to_f64(ref["h"], BF16))))
    y = moe.moe_grouped_gemm_w2(act_to_torch(ref["h"], mode), D["w2"], D["w2_scale"],
                                int_tensor(ref["offsets"]), f32_tensor(act), k)
    torch.cuda.synchronize()
    y_ref, _ = oracle.w2(mode, ref["h"], L["w2"], L["w2_scale"], ref["offsets"], k)
    assert rel_inf(y.cpu().numpy(), y_ref) <= (2e-4 if mode == FP8 else 1e-5)


@pytest.mark.parametrize("c", [CASES[3], CASES[7], CASES[14], CASES[19]],
                         ids=["bf16_small", "fp8_zipf", "fp8_tiles_ragged", "fp8_chunked_sort"])
def test_fused_forward_full_softmax_weights(c):
    # renormalize = 0: the selected experts keep their full-softmax
    # probabilities (through every front-end path: one-block, per-expert
    # grouping, chunked sort)
    name, T, H, E, k, I, mode, routing = c
    L, _ = case(c)
    ref = oracle.forward(mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"],
                         L["w2_scale"], k, renormalize=False)
    D = upload(L)
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    say("fused renormalize=0", name)
    out = moe.moe_fused_forward(D["x"], D["logits"], D["w13"], D["w13_scale"], D["w2"],
                                D["w2_scale"], k, renormalize=False, topk_weights=w)
    torch.cuda.synchronize()
    assert np.max(np.abs(w.cpu().numpy() - ref["topk_weights"])) <= 1e-6
    err = rel_inf(oracle.to_f64(act_to_numpy(out, mode), mode), ref["out_exact"])
    say("  rel err", err)
    assert err <= OUT_TOL[mode]


@pytest.mark.parametrize("c", [c for c in CASES if c[6] == FP8 and c[1] * c[4] >= 16 * c[3]],
                         ids=lambda c: c[0])
def test_fused_fp8_tiles_equals_steps(c):
    """FP8 layers with many pairs per expert: the fused call keeps y in bf16
    between the down projection and the aggregation.  Its output equals the
    step entry points' (same kernels, same order) once the step API's fp32 y
    is rounded to bf16 (nearest even) before moe_combine."""
    name, T, H, E, k, I, mode, routing = c
    L, ref = case(c)
    D = upload(L)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    say("fused vs steps", name)
    out = moe.moe_fused_forward(D["x"], D["logits"], D["w13"], D["w13_scale"], D["w2"],
                                D["w2_scale"], k, topk_ids=ids, topk_weights=w)
    counts, offsets, sorted_ids, inv = moe.moe_align_sort(ids, E)
    h, sc = moe.moe_grouped_gemm_w13_swiglu(D["x"], D["w13"], D["w13_scale"], sorted_ids, offsets,
                                            k)
    y = moe.moe_grouped_gemm_w2(h, D["w2"], D["w2_scale"], offsets, sc, k)
    y_b = y.to(torch.bfloat16).to(torch.float32)
    out_steps = moe.moe_combine(y_b, inv, w, mode, E=E)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_steps.view(torch.int16))


def _random_shapes(n, seed=2024):
    """Seeded layer shapes within the interface's limits, across the shape
    classes: one-block and many-pair fronts, few-token and tiled GEMMs
    (64- and 128-position tiles), every mode and routing recipe."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mode = int(rng.integers(0, 3))
        E = int(rng.choice([1, 3, 8, 17, 32, 64, 100]))
        k = int(rng.integers(1, min(E, 16) + 1))
        T = int(rng.choice([1, 5, 33, 100, 257, 600, 1500]))
        H = 128 * int(rng.integers(1, 4))
        I = 128 * int(rng.integers(1, 5))
        routing = str(rng.choice(["uniform", "zipf", "empty"])) if E >= 10 else "uniform"
        out.append(("rand%02d" % i, T, H, E, k, I, mode, routing))
    return out


RANDOM = _random_shapes(24)


@pytest.mark.parametrize("c", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_shape_sweep(c):
    name, T, H, E, k, I, mode, routing = c
    L = wl.make_layer(wl.scaled(name, T, H, E, k, I, mode, routing=routing, seed=7 + len(name)))
    ref = oracle.forward(mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"],
                         L["w2_scale"], k)
    D = upload(L)
    out = torch.full((T, H), float("nan"), dtype=moe.act_dtype(mode), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    say("random shape", c)
    _, grp = fused_call(D, k, mode, out=out, topk_ids=ids)
    assert np.array_equal(ids.cpu().numpy(), ref["topk_ids"])
    assert_grouping(grp, ref["counts"], ref["offsets"], ref["sorted_ids"], ref["inv_perm"])
    og = oracle.to_f64(act_to_numpy(out, mode), mode)
    assert not np.isnan(og).any()
    err = rel_inf(og, ref["out_exact"])
    say("  rel err", err)
    assert err <= OUT_TOL[mode]
