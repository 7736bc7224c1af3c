"""Pins for the oracle's number codecs (bf16 RNE, OCP e4m3fn) -- CPU only.

The oracle's codecs are checked against things other than themselves:
hand-derived values from the format definitions (tests/golden), exhaustive
brute-force nearest-even search, and PyTorch's own dtype conversions.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _finite_e4m3_table():
    """All finite e4m3 values via PyTorch's decoder (a library routine)."""
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = ~np.isnan(vals)
    return codes[finite], vals[finite]


def test_e4m3_decode_golden():
    d = json.load(open(os.path.join(GOLDEN, "e4m3_ocp_values.json")))
    for code_s, val_s in d["decode"]:
        got = oracle.e4m3_decode(np.array([int(code_s, 16)], np.uint8))[0]
        if val_s == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val_s), (code_s, got)


def test_e4m3_encode_golden():
    d = json.load(open(os.path.join(GOLDEN, "e4m3_ocp_values.json")))
    vals = np.array([float(v) for v, _, _ in d["encode"]], np.float32)
    want = np.array([int(c, 16) for _, c, _ in d["encode"]], np.uint8)
    got = oracle.e4m3_encode(vals)
    bad = [(d["encode"][i][0], hex(got[i]), d["encode"][i][1]) for i in np.nonzero(got != want)[0]]
    assert not bad, bad


def test_e4m3_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2  # only S.1111.111


def test_e4m3_encode_every_bf16_bruteforce():
    """Every one of the 65536 bf16 patterns -> nearest-even e4m3 by search."""
    bits = np.arange(65536, dtype=np.uint32)
    v32 = (bits << 16).view(np.float32)
    v32 = v32[~np.isnan(v32)]
    got = oracle.e4m3_encode(v32)
    codes, vals = _finite_e4m3_table()
    # brute force: distance to every finite value, saturating beyond +-448
    x = np.clip(v32.astype(np.float64), -448.0, 448.0)
    dist = np.abs(x[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among equidistant candidates keep the one with an even code (lsb 0)
    even = (codes & 1) == 0
    pick_even = cand & even[None, :]
    has_even = pick_even.any(axis=1)
    choice = np.where(has_even, np.argmax(pick_even, axis=1), np.argmax(cand, axis=1))
    want = codes[choice]
    # the sign of zero follows the input
    zero = vals[choice] == 0
    want = np.where(zero, np.where(np.signbit(v32), 0x80, 0x00), want).astype(np.uint8)
    mism = np.nonzero(got != want)[0]
    assert mism.size == 0, [(float(v32[i]), hex(got[i]), hex(want[i])) for i in mism[:10]]


def test_e4m3_encode_random_fp32_vs_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 100,
        rng.standard_normal(200000).astype(np.float32) * 0.01,
        (rng.uniform(-500, 500, 100000)).astype(np.float32),
    ])
    got = oracle.e4m3_encode(v)
    ref = torch.from_numpy(v).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps -0 for tiny negatives as we do
    assert np.array_equal(got, ref)


def test_bf16_round_golden():
    d = json.load(open(os.path.join(GOLDEN, "bf16_rne_values.json")))
    vals = np.array([float(r[0]) for r in d["round"]], np.float64)
    want = np.array([int(r[1], 16) for r in d["round"]], np.uint16)
    got = oracle.bf16_round(vals)
    assert np.array_equal(got, want), list(zip(vals, [hex(g) for g in got]))


def test_bf16_round_fp32_inputs_vs_torch():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.standard_normal(300000).astype(np.float32),
        rng.standard_normal(100000).astype(np.float32) * 1e-30,
        rng.standard_normal(100000).astype(np.float32) * 1e30,
        ((np.arange(65536, dtype=np.uint32) << 16) | 0x8000).view(np.float32),  # exact ties
    ])
    v = v[np.isfinite(v)]
    got = oracle.bf16_round(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_round_double_inputs_exact():
    """Double inputs between two bf16 neighbours: nearest, ties to even (exact search)."""
    rng = np.random.default_rng(3)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    got = oracle.bf16_round(v)
    gv = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # neighbours: truncate toward zero in fp32 bits and the next bf16 up in magnitude
    f32 = v.astype(np.float32)  # only used to find a nearby bf16 pattern
    base = (f32.view(np.uint32) & 0xFFFF0000).astype(np.uint32)
    cands = []
    for d in (-1, 0, 1, 2):
        b = (base.astype(np.int64) + d * 0x10000).astype(np.uint32)
        cands.append(b.view(np.float32).astype(np.float64))
    C = np.stack(cands, 1)
    dist = np.abs(C - v[:, None])
    best = dist.min(1)
    assert np.all(np.abs(gv - v) == best)
    # ties (not expected for random doubles, but checked) must land on an even pattern
    ntie = ((dist == best[:, None]).sum(1) > 1)
    assert np.all((got[ntie] & 1) == 0)
