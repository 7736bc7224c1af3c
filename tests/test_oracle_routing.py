"""Pins for the oracle's gating and grouping steps -- CPU only.

Checked against a library stable sort (ties keep the lower index), the full
float64 softmax restricted to the selected experts, hand-worked closed forms
(tests/golden/gating_closed_form.json) and the grouping invariants.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import BF16, F32
from oracle import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(s):
    return float(eval(s, {"exp": math.exp, "inf": math.inf}))


def _logits(rng, T, E, kind):
    if kind == "normal":
        return rng.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":  # few distinct values -> many exact ties
        return rng.integers(-2, 3, (T, E)).astype(np.float32)
    if kind == "neginf":
        l = rng.standard_normal((T, E)).astype(np.float32)
        l[rng.random((T, E)) < 0.4] = -np.inf
        return l
    if kind == "signed_zero":
        l = rng.choice(np.array([0.0, -0.0, -1.0], np.float32), (T, E))
        return l.astype(np.float32)
    raise ValueError(kind)


def test_gating_golden_closed_form():
    d = json.load(open(os.path.join(GOLDEN, "gating_closed_form.json")))
    for c in d["cases"]:
        l = np.array([[_ev(v) for v in c["logits"]]], np.float32)
        ids, w = oracle.topk_gating(l, c["k"], bool(c["renormalize"]))
        assert ids[0].tolist() == c["ids"]
        want = np.array([_ev(v) for v in c["weights"]])
        assert np.max(np.abs(w[0] - want)) <= 1e-7, (w[0], want)


@pytest.mark.parametrize("kind", ["normal", "ties", "neginf", "signed_zero"])
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (37, 8, 2), (50, 64, 8), (9, 256, 8), (5, 16, 16)])
def test_gating_vs_stable_sort_and_softmax(kind, T, E, k):
    rng = np.random.default_rng(T * 1000 + E + k)
    l = _logits(rng, T, E, kind)
    if kind == "neginf":  # keep >= k finite entries per row (precondition)
        for t in range(T):
            fin = np.isfinite(l[t])
            if fin.sum() < k:
                l[t, :k] = rng.standard_normal(k).astype(np.float32)
    for renorm in (True, False):
        ids, w = oracle.topk_gating(l, k, renorm)
        ref_ids, ref_w = bf.routing(l, k, renorm)
        assert np.array_equal(ids, ref_ids)
        assert np.max(np.abs(w.astype(np.float64) - ref_w)) <= 1e-6
        if renorm:
            assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 1e-6)
        # selected ids are distinct and in range
        assert all(len(set(r)) == k for r in ids.tolist())
        assert ids.min() >= 0 and ids.max() < E


def test_gating_all_equal():
    l = np.full((4, 8), 0.25, np.float32)
    ids, w = oracle.topk_gating(l, 3)
    assert np.array_equal(ids, np.tile(np.arange(3), (4, 1)))
    assert np.allclose(w, 1.0 / 3.0, rtol=0, atol=1e-7)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (16, 8, 2), (128, 64, 8), (333, 256, 8), (7, 1, 1)])
def test_grouping_vs_library_and_invariants(T, E, k):
    rng = np.random.default_rng(T + E)
    l = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.topk_gating(l, k)
    counts, offsets, sorted_ids, inv = oracle.align_sort(ids, E)
    rc, ro, rs, ri = bf.grouping(ids, E)
    assert np.array_equal(counts, rc)
    assert np.array_equal(offsets, ro)
    assert np.array_equal(sorted_ids, rs)
    assert np.array_equal(inv, ri)
    # invariants
    n = T * k
    assert counts.sum() == n
    assert offsets[0] == 0 and offsets[E] == n and np.all(np.diff(offsets) >= 0)
    assert np.array_equal(np.sort(sorted_ids), np.arange(n))
    assert np.array_equal(np.bincount(sorted_ids // k, minlength=T), np.full(T, k))
    assert np.array_equal(sorted_ids[inv], np.arange(n))
    flat = ids.ravel()
    for e in range(E):
        seg = sorted_ids[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0)  # stable: ascending pair index


def test_grouping_skewed_and_empty():
    E, T, k = 32, 64, 4
    ids = np.zeros((T, k), np.int32)
    for t in range(T):  # everything on experts 3,4,5,6 -> 28 empty experts
        ids[t] = [3, 4, 5, 6]
    counts, offsets, sorted_ids, inv = oracle.align_sort(ids, E)
    assert counts[3] == T and counts[0] == 0 and counts[31] == 0
    assert np.array_equal(sorted_ids[:T], np.arange(T) * k)
    assert offsets[4] == T and offsets[E] == T * k


# ------------------------------------------------------------ router logits
def _to_act(a, mode):
    a = np.ascontiguousarray(a, np.float32)
    return a if mode == F32 else oracle.bf16_round(a.astype(np.float64)).reshape(a.shape)


@pytest.mark.parametrize("mode", [F32, BF16])
def test_router_logits_integer_inputs_exact(mode):
    # small integers are exact in bf16 and their dot products are exact
    # integers: the logits are known exactly (int64 matmul, a different code
    # path from the oracle's double loop)
    rng = np.random.default_rng(4)
    T, H, E = 7, 96, 5
    xi = rng.integers(-8, 9, (T, H))
    wi = rng.integers(-8, 9, (E, H))
    got = oracle.router_logits(mode, _to_act(xi, mode), _to_act(wi, mode))
    assert got.dtype == np.float32 and got.shape == (T, E)
    assert np.array_equal(got, (xi @ wi.T).astype(np.float32))


@pytest.mark.parametrize("mode", [F32, BF16])
def test_router_logits_unit_vectors_pick_weights(mode):
    # x = unit vector e_h  ->  logits[:, e] = wg[e, h]: pins the orientation
    # (wg holds one row per expert) and the indexing of both operands
    rng = np.random.default_rng(5)
    H, E = 24, 6
    wg = _to_act(rng.standard_normal((E, H)).astype(np.float32), mode)
    x = _to_act(np.eye(H, dtype=np.float32), mode)
    got = oracle.router_logits(mode, x, wg)
    assert np.array_equal(got, oracle.to_f64(wg, mode).T.astype(np.float32))


def test_router_logits_random_bf16_vs_float64_matmul():
    # products of bf16 values are exact in double and, at these magnitudes,
    # so are their sums: any summation order gives the same double
    rng = np.random.default_rng(6)
    T, H, E = 33, 512, 40
    x = _to_act(rng.standard_normal((T, H)), BF16)
    wg = _to_act(0.02 * rng.standard_normal((E, H)), BF16)
    ref = (oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(wg).T).astype(np.float32)
    assert np.array_equal(oracle.router_logits(BF16, x, wg), ref)
