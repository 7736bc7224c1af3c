"""GPU parity at the full layer sizes, in the launch configuration bench.py
times (one moe_fused_forward call per layer), called through the C ABI.

Routing (top-k ids, counts, offsets, sorted ids, inverse permutation) and the
FP8 activation scale s_x are bit-exact against the CPU oracle everywhere; the
grouping compared is the one the fused call's own kernels wrote into its
workspace (the one-block front kernel for the decode layers, one block per
expert for the mixed layer, the chunked counting sort for the prefill
layers).

* decode layers (bf16 T=8; FP8 T=1, 4, 16) and the mixed FP8 layer: the
  oracle computes the whole layer, so `out` is compared element by element
  (max|gpu - ref| / max|ref| <= 5e-3 bf16, 2e-2 FP8, ref = the oracle's
  output before its final rounding to bf16).
* prefill FP8 layers (4096 tokens, and 16384 tokens for the compute-bound
  regime; 256 experts): the oracle's cost (about 1e12 multiply-adds for h
  alone at 4096 tokens) rules out the whole layer, so it checks
  sampled h rows (first, last and ragged-tail rows of the heaviest experts,
  single-pair experts), the exact amax(h) of the GPU's own h, the output
  of sampled tokens (down projection and aggregation run by the oracle on
  the GPU's own h, whose e4m3 codes are decided on it), and that the
  fused call's output equals the step-by-step entry points' output bit for
  bit (with the step API's fp32 y rounded to bf16, as the fused FP8 path of
  many-token layers keeps it).  A prefill-shaped slice (H=7168, I=2048,
  k=8, Zipf skew, 32 experts, 512 tokens: the same 128-position tiled
  kernels and K extents) is then compared element by element with the
  oracle.
"""
import numpy as np
import pytest
import torch

import moe_layer_gating_amd as moe
import moe_workloads as wl
import oracle
from gpu_helpers import (BF16, FP8, OUT_TOL, act_to_numpy, assert_grouping, bf16_step_ratio,
                         fused_call, h_identical_min, int_tensor, rel_inf, say, upload)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()


def _gen(spec):
    say("generating", spec.name, "T=%d H=%d E=%d k=%d I=%d" % (spec.T, spec.H, spec.E, spec.k,
                                                                 spec.I))
    return wl.make_layer(spec)


def _fused(D, k, T, H, mode):
    out = torch.full((T, H), float("nan"), dtype=moe.act_dtype(mode), device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    _, grp = fused_call(D, k, mode, out=out, topk_ids=ids, topk_weights=w)
    return out, ids.cpu().numpy(), w.cpu().numpy(), grp


def _check_routing(L, ids, w, grp, k, E):
    """ids and weights against the oracle's gating, and the grouping the
    fused call wrote against the oracle's grouping, bit for bit."""
    rid, rw = oracle.topk_gating(L["logits"], k)
    assert np.array_equal(ids, rid), "top-k ids differ"
    assert np.max(np.abs(w - rw)) <= 1e-6
    rc, ro, rs, ri = oracle.align_sort(rid, E)
    assert_grouping(grp, rc, ro, rs, ri)
    return rc, ro, rs, ri


def _full_layer(L, D, mode):
    s = L["spec"]
    out, ids, w, grp = _fused(D, s.k, s.T, s.H, mode)
    _check_routing(L, ids, w, grp, s.k, s.E)
    say("  oracle forward")
    ref = oracle.forward(mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"],
                         L["w2_scale"], s.k)
    og = oracle.to_f64(act_to_numpy(out, mode), mode)
    assert not np.isnan(og).any(), "an output row was not written"
    err = rel_inf(og, ref["out_exact"])  # the oracle's output before its final rounding
    say("  %s: rel err %.3g (tolerance %g)" % (s.name, err, OUT_TOL[mode]))
    assert err <= OUT_TOL[mode]


def test_decode_bf16_full():
    L = _gen(wl.WORKLOADS["decode_bf16"])
    _full_layer(L, upload(L), BF16)


def test_decode_fp8_full_t1_t4_t16():
    # one weight set for T = 1, 4, 16; x and logits are the first T rows of
    # the 16-row draw (the generator's recipe for these layers)
    L16 = _gen(wl.WORKLOADS["decode_fp8_t16"])
    D16 = upload(L16)
    for T in (1, 4, 16):
        spec = wl.WORKLOADS["decode_fp8_t%d" % T]
        L = dict(L16, spec=spec, x=L16["x"][:T].copy(), logits=L16["logits"][:T].copy())
        D = dict(D16, x=D16["x"][:T].contiguous(), logits=D16["logits"][:T].contiguous())
        say(" T =", T)
        _full_layer(L, D, FP8)


def test_mixed_fp8_full():
    L = _gen(wl.WORKLOADS["mixed_fp8"])
    s = L["spec"]
    D = upload(L)
    _full_layer(L, D, FP8)
    # the 13 experts whose logits are -inf receive no pairs
    dead = np.where(np.all(np.isneginf(L["logits"]), axis=0))[0]
    assert dead.size == round(0.1 * s.E)


def _sample_positions(counts, offsets, rng):
    """First, last and ragged-tail rows of the heaviest experts, every
    single-pair expert's row, plus random rows."""
    pos = set()
    order = np.argsort(-counts, kind="stable")
    for e in order[:6]:
        a, b = offsets[e], offsets[e + 1]
        if b > a:
            pos.update([a, b - 1, a + (b - a) // 2])
            tail = a + ((b - a - 1) // 128) * 128  # first row of the last 128-row tile
            pos.update([tail, min(tail + 1, b - 1)])
    pos.update(offsets[:-1][counts == 1].tolist())
    pos.update(rng.integers(0, offsets[-1], 24).tolist())
    return np.array(sorted(pos), np.int64)


@pytest.mark.parametrize("name", ["prefill_fp8", "prefill_fp8_t16k"])
def test_prefill_fp8_full_sampled(name):
    L = _gen(wl.WORKLOADS[name])
    s = L["spec"]
    D = upload(L)
    out, ids, w, grp = _fused(D, s.k, s.T, s.H, FP8)
    rc, ro, rs, ri = _check_routing(L, ids, w, grp, s.k, s.E)
    og = act_to_numpy(out, FP8)
    assert not np.isnan(oracle.to_f64(og, FP8)).any()
    say("  step API")
    sorted_t, off_t = int_tensor(rs), int_tensor(ro)
    h, sc = moe.moe_grouped_gemm_w13_swiglu(D["x"], D["w13"], D["w13_scale"], sorted_t, off_t,
                                            s.k)
    y = moe.moe_grouped_gemm_w2(h, D["w2"], D["w2_scale"], off_t, sc, s.k)
    # the fused call keeps y in bf16 (FP8, many tokens per expert): the same
    # y rounded to nearest even, then the same aggregation
    y_b = y.to(torch.bfloat16).to(torch.float32)
    out_steps = moe.moe_combine(y_b, int_tensor(ri), torch.from_numpy(w).cuda(), FP8, E=s.E)
    torch.cuda.synchronize()
    # the fused call and the step entry points run the same kernels
    assert np.array_equal(act_to_numpy(out_steps, FP8), og)
    scales = sc.cpu().numpy()
    hg = act_to_numpy(h, FP8)
    _, s_x, _ = oracle.act_quant(L["x"], BF16)
    assert scales[0] == s_x
    hv = oracle.to_f64(hg, FP8)
    assert scales[3] == np.float32(np.max(np.abs(hv)))
    assert scales[1] == np.float32(scales[3]) / np.float32(448.0)
    pos = _sample_positions(rc, ro, np.random.default_rng(3))
    say("  oracle h rows:", len(pos))
    href, _ = oracle.w13_swiglu(FP8, L["x"], L["w13"], L["w13_scale"], rs, ro, s.k,
                                positions=pos)
    ratio = bf16_step_ratio(hv[pos], oracle.to_f64(href, FP8))
    say("  sampled h: step ratio %.3f, identical %.4f" % (ratio, np.mean(hg[pos] == href)))
    assert ratio <= 1.0
    assert np.mean(hg[pos] == href) >= h_identical_min(FP8, s.T, s.k, s.E)
    # down projection and aggregation of sampled tokens at full size, from
    # the GPU's own h (the e4m3 codes of h are decided on it, with the scale
    # of its amax, checked above): tokens of the heaviest expert's first and
    # last rows, of single-pair experts, and random tokens
    rng = np.random.default_rng(5)
    toks = set(rng.integers(0, s.T, 16).tolist())
    e_max = int(np.argmax(rc))
    toks.update([int(rs[ro[e_max]]) // s.k, int(rs[ro[e_max + 1] - 1]) // s.k])
    toks.update(int(rs[ro[e]]) // s.k for e in np.where(rc == 1)[0][:4])
    toks = np.array(sorted(toks), np.int64)
    pairs = (toks[:, None] * s.k + np.arange(s.k)[None, :]).ravel()
    say("  oracle down projection + aggregation of %d tokens" % len(toks))
    y_s, s_h = oracle.w2(FP8, hg, L["w2"], L["w2_scale"], ro, s.k, positions=ri[pairs])
    assert s_h == scales[1]
    _, o_ref = oracle.combine(FP8, y_s, np.arange(pairs.size, dtype=np.int32), w[toks],
                              exact=True)
    err = rel_inf(oracle.to_f64(og[toks], FP8), o_ref)
    say("  sampled out: rel err %.3g (tolerance %g)" % (err, OUT_TOL[FP8]))
    assert err <= OUT_TOL[FP8]


def test_prefill_shaped_slice_full():
    spec = wl.scaled("prefill_slice", 512, 7168, 32, 8, 2048, FP8, routing="zipf", seed=11)
    L = _gen(spec)
    _full_layer(L, upload(L), FP8)
