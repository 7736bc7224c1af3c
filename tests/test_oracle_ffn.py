"""Pins for the oracle's expert FFN, quantisation and combine -- CPU only.

The per-token oracle loop is checked against: a dense brute-force evaluation
of every expert masked by the top-k choice (oracle/bruteforce.py), a dense
SwiGLU MLP computed with PyTorch (E=1, k=1), the full softmax mixture (k=E),
hand-worked closed forms (tests/golden/ffn_tiny_closed_form.json), x = 0, and
PyTorch / NumPy for the per-tensor FP8 quantiser.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_workloads as wl
import oracle
from oracle import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32, BF16, FP8 = oracle.F32, oracle.BF16, oracle.FP8


def _ev(s):
    return float(eval(s, {"exp": math.exp}))


def _rel_inf(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return np.max(np.abs(a - b)) / (den if den > 0 else 1.0)


def _layer(T, H, E, k, I, mode, routing="uniform", seed=0):
    return wl.make_layer(wl.scaled("t", T, H, E, k, I, mode, routing=routing, seed=seed))


def _run_both(L, renorm=True):
    s = L["spec"]
    o = oracle.forward(s.mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"], L["w2_scale"],
                       s.k, renorm)
    b = bf.forward(s.mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"], L["w2_scale"],
                   s.k, renorm)
    return oracle.to_f64(o["out"], s.mode), b, o


def test_golden_tiny_ffn_closed_form():
    d = json.load(open(os.path.join(GOLDEN, "ffn_tiny_closed_form.json")))
    x = np.array(d["x"], np.float32)
    w13 = np.array(d["w13"], np.float32)
    w2 = np.array(d["w2"], np.float32)
    lg = np.array(d["logits"], np.float32)
    for c in d["cases"]:
        r = oracle.forward(F32, x, lg, w13, None, w2, None, c["k"])
        assert r["topk_ids"].tolist() == c["ids"]
        want = np.array([[_ev(e) for e in row] for row in c["out"]])
        assert np.max(np.abs(r["out"] - want)) <= 1e-6, (r["out"], want)


@pytest.mark.parametrize("mode", [F32, BF16, FP8])
@pytest.mark.parametrize("shape", [(7, 32, 6, 3, 24), (16, 64, 8, 2, 40), (3, 48, 4, 4, 16)])
def test_oracle_vs_bruteforce(mode, shape):
    T, H, E, k, I = shape
    L = _layer(T, H, E, k, I, mode, seed=sum(shape) + mode)
    for renorm in (True, False):
        o, b, _ = _run_both(L, renorm)
        tol = {F32: 1e-6, BF16: 8e-3, FP8: 8e-3}[mode]
        err = _rel_inf(o, b)
        assert err <= tol, err
        if mode != F32:
            # output rounding aside, almost every element agrees exactly
            assert np.mean(o == b) > 0.97


def test_oracle_vs_bruteforce_tiny_f32_workload():
    """The 16-token fp32 layer (hidden 128, 8 experts, top-2, I=256) at full size."""
    L = wl.make_layer(wl.WORKLOADS["tiny_f32"])
    o, b, r = _run_both(L)
    assert _rel_inf(o, b) <= 1e-6
    ids, _ = bf.routing(L["logits"], 2)
    assert np.array_equal(r["topk_ids"], ids)


def test_zipf_and_empty_routing_shapes():
    L = _layer(64, 32, 16, 4, 16, FP8, routing="zipf", seed=5)
    o, b, r = _run_both(L)
    assert _rel_inf(o, b) <= 8e-3
    assert r["counts"].max() > 2 * r["counts"].mean()  # skewed load
    L = _layer(40, 32, 20, 4, 16, FP8, routing="empty", seed=6)
    o, b, r = _run_both(L)
    assert _rel_inf(o, b) <= 8e-3
    assert (r["counts"] == 0).sum() >= 2  # round(0.1*20) experts forced empty


def test_single_expert_is_dense_swiglu_mlp():
    """E=1, k=1: the layer is a dense SwiGLU MLP (PyTorch float64)."""
    T, H, I = 9, 40, 24
    L = _layer(T, H, 1, 1, I, F32, seed=11)
    r = oracle.forward(F32, L["x"], L["logits"], L["w13"], None, L["w2"], None, 1)
    x = torch.from_numpy(L["x"]).double()
    w13 = torch.from_numpy(L["w13"][0]).double()
    w2 = torch.from_numpy(L["w2"][0]).double()
    g = torch.nn.functional.linear(x, w13[:I])
    u = torch.nn.functional.linear(x, w13[I:])
    ref = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, w2).numpy()
    assert np.max(np.abs(r["out"] - ref)) <= 1e-6 * np.max(np.abs(ref))
    assert np.allclose(r["topk_weights"], 1.0)


def test_k_equals_E_is_full_softmax_mixture():
    """k = E with renormalisation: the mixture weights are the full softmax."""
    T, H, E, I = 5, 24, 4, 16
    L = _layer(T, H, E, E, I, F32, seed=12)
    r = oracle.forward(F32, L["x"], L["logits"], L["w13"], None, L["w2"], None, E)
    x = torch.from_numpy(L["x"]).double()
    p = torch.softmax(torch.from_numpy(L["logits"]).double(), dim=1)
    out = torch.zeros(T, H, dtype=torch.float64)
    for e in range(E):
        w13 = torch.from_numpy(L["w13"][e]).double()
        w2 = torch.from_numpy(L["w2"][e]).double()
        hh = torch.nn.functional.silu(x @ w13[:I].T) * (x @ w13[I:].T)
        out += p[:, e:e + 1] * (hh @ w2.T)
    assert np.max(np.abs(r["out"] - out.numpy())) <= 1e-6 * float(out.abs().max())


@pytest.mark.parametrize("mode", [F32, BF16, FP8])
def test_zero_input_gives_zero_output(mode):
    L = _layer(6, 32, 4, 2, 16, mode, seed=13)
    x = np.zeros_like(L["x"])
    r = oracle.forward(mode, x, L["logits"], L["w13"], L["w13_scale"], L["w2"], L["w2_scale"], 2)
    assert np.all(oracle.to_f64(r["out"], mode) == 0.0)
    if mode == FP8:
        assert r["scales"][0] == 1.0 and r["scales"][1] == 1.0  # amax 0 -> scale 1


def test_act_quant_vs_numpy_and_torch():
    rng = np.random.default_rng(4)
    x32 = rng.standard_normal((37, 300)).astype(np.float32) * 3
    xb = wl.to_bf16_bits(x32)
    codes, s, r = oracle.act_quant(xb, BF16)
    vals = wl.bf16_bits_values(xb)
    A = np.float32(np.max(np.abs(vals)))
    assert s == np.float32(A) / np.float32(448.0)
    assert r == np.float32(448.0) / np.float32(A)
    prod = (vals * r).astype(np.float32)
    ref = torch.from_numpy(prod).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref)
    # the element holding the maximum lands on +-448 up to one rounding of A * r
    i = np.argmax(np.abs(vals))
    assert abs(oracle.e4m3_decode(codes.ravel()[i:i + 1])[0]) == 448.0


@pytest.mark.parametrize("mode", [F32, BF16, FP8])
def test_steps_compose_to_forward(mode):
    """The step functions (gating, sort, w13, w2, combine) reproduce forward()."""
    T, H, E, k, I = 11, 32, 6, 3, 24
    L = _layer(T, H, E, k, I, mode, seed=14)
    r = oracle.forward(mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"], L["w2_scale"], k)
    ids, w = oracle.topk_gating(L["logits"], k)
    counts, offsets, sorted_ids, inv = oracle.align_sort(ids, E)
    h, s_x = oracle.w13_swiglu(mode, L["x"], L["w13"], L["w13_scale"], sorted_ids, offsets, k)
    assert np.array_equal(h, r["h"])
    y, s_h = oracle.w2(mode, h, L["w2"], L["w2_scale"], offsets, k)
    out = oracle.combine(mode, y, inv, w)
    assert np.array_equal(out, r["out"])
    # sampled positions give the same rows as the full computation
    pos = np.array([0, 5, T * k - 1])
    hs, _ = oracle.w13_swiglu(mode, L["x"], L["w13"], L["w13_scale"], sorted_ids, offsets, k,
                              positions=pos)
    assert np.array_equal(hs, h[pos])
    ys, _ = oracle.w2(mode, h, L["w2"], L["w2_scale"], offsets, k, positions=pos)
    assert np.array_equal(ys, y[pos])


@pytest.mark.parametrize("mode", [F32, BF16, FP8])
def test_out_is_the_rounding_of_out_exact(mode):
    """The stored output is the output type's rounding of out_exact."""
    L = _layer(9, 64, 8, 2, 48, mode, seed=4 + mode)
    s = L["spec"]
    r = oracle.forward(mode, L["x"], L["logits"], L["w13"], L["w13_scale"], L["w2"], L["w2_scale"],
                       s.k)
    if mode == F32:
        assert np.array_equal(r["out"], r["out_exact"].astype(np.float32))
    else:
        assert np.array_equal(r["out"].ravel(), bf.f64_to_bf16_values(r["out_exact"]).astype(
            np.float32).view(np.uint32).ravel().__rshift__(16).astype(np.uint16))


def _ulp(v, mode):
    """Spacing of the output type at |v| (fp32, or bf16 in the other modes)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return np.exp2(e - (23 if mode == F32 else 7))


@pytest.mark.parametrize("mode", [F32, BF16])
@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 3, 5), (33, 8, 64), (16, 16, 16)])
def test_combine_f32_pins(mode, T, k, E):
    """oracle_combine_f32 (the expected value of the GPU combine stage test),
    pinned three ways on fp32 y in sorted order:
      * the double-precision oracle_combine on the same y widened to double
        (exact widening: identical sums, identical results);
      * a dense mixing matrix M[t, inv_perm[t*k+j]] = w[t,j] applied with a
        float64 matmul (a different construction: a wrong index, a swapped
        weight or a dropped slot changes it by far more than the one output
        ulp that the summation order may move);
      * special cases: k = 1 with weight 1 is an exact gather of y's rows;
        equal weights on equal rows return that row."""
    rng = np.random.default_rng(T * 100 + k * 10 + E)
    H = 24
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    _, _, sorted_ids, inv = oracle.align_sort(ids, E)
    y = rng.standard_normal((T * k, H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    got = oracle.to_f64(oracle.combine(mode, y, inv, w), mode)
    want_dd = oracle.to_f64(oracle.combine(mode, y.astype(np.float64), inv, w), mode)
    assert np.array_equal(got, want_dd)
    M = np.zeros((T, T * k))
    for t in range(T):
        for j in range(k):
            M[t, inv[t * k + j]] += w[t, j]
    dense = M @ y.astype(np.float64)
    assert np.all(np.abs(got - dense) <= _ulp(dense, mode))
    # k = 1, weight 1: out is y gathered by inv_perm, exactly (bf16: rounded once)
    if k == 1:
        g1 = oracle.to_f64(oracle.combine(mode, y, inv, np.ones((T, 1), np.float32)), mode)
        gather = y.astype(np.float64)[inv]
        if mode == F32:
            assert np.array_equal(g1, gather)
        else:
            assert np.array_equal(g1, oracle.to_f64(oracle.bf16_round(gather), BF16).reshape(T, H))
    # equal weights on equal rows: the row itself
    row = rng.standard_normal(H).astype(np.float32)
    ysame = np.tile(row, (T * k, 1))
    wq = np.full((T, k), np.float32(1.0 / k), np.float32) if k in (1, 2, 8, 16) else None
    if wq is not None:  # 1/k exact in fp32, sums of k equal terms exact
        g2 = oracle.to_f64(oracle.combine(mode, ysame, inv, wq), mode)
        r = row.astype(np.float64)[None, :].repeat(T, 0)
        if mode == F32:
            assert np.array_equal(g2, r)
        else:
            assert np.array_equal(g2, oracle.to_f64(oracle.bf16_round(r), BF16).reshape(T, H))
