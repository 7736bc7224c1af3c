"""Pins for the oracle's inverse rotary embedding + per-head FP8 quantisation
(oracle.inv_rope_fp8) -- CPU only.

The rotation is checked against: the identity at angle 0, an exact quarter
turn, a dense rotation-matrix product in float64 (a different construction:
a wrong pair index, sign, forward-for-inverse or transposed table fails it),
norm preservation, and a hand-worked example (tests/golden/). The per-head
quantisation is checked through the dequantisation error bound, the largest
element landing on the largest code, and the zero-head rule; the e4m3 codec
itself is pinned exhaustively in test_oracle_codecs.py.
"""
import json
import os

import numpy as np
import pytest

import oracle
from moe_workloads import to_bf16_bits, bf16_bits_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24


def _x(rng, T, nh, hd, sigma=1.0):
    return to_bf16_bits((rng.standard_normal((T, nh, hd)) * sigma).astype(np.float32)).reshape(
        T, nh, hd)


def _table(max_pos, rot, base=10000.0):
    half = rot // 2
    theta = base ** (-2.0 * np.arange(half) / rot)
    ang = np.arange(max_pos)[:, None] * theta[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def _pairs(hd, rot, inter):
    half = rot // 2
    return [(2 * i, 2 * i + 1) if inter else (i, i + half) for i in range(half)]


def test_golden_hand_worked():
    d = json.load(open(os.path.join(GOLDEN, "inv_rope_fp8_hand.json")))
    x = to_bf16_bits(np.array(d["x"], np.float32)).reshape(1, 1, 4)
    cs = np.array([d["cos"] + d["sin"]], np.float32)
    for c in d["cases"]:
        codes, sc, y = oracle.inv_rope_fp8(x, np.zeros(1, np.int32), cs,
                                           interleaved=c["interleaved"])
        assert y.ravel().tolist() == c["y"]
        assert sc[0, 0] == np.float32(np.float32(c["amax"]) / np.float32(448.0))
        assert [format(v, "02x") for v in codes.ravel()] == c["codes_hex"]
        assert oracle.e4m3_decode(codes.ravel()).tolist() == c["code_values"]


@pytest.mark.parametrize("inter", [0, 1])
def test_angle_zero_is_identity(inter):
    rng = np.random.default_rng(1)
    x = _x(rng, 5, 3, 64)
    cs = _table(16, 64)
    _, _, y = oracle.inv_rope_fp8(x, np.zeros(5, np.int32), cs, interleaved=inter)
    assert np.array_equal(y, bf16_bits_values(x).reshape(y.shape))


@pytest.mark.parametrize("inter", [0, 1])
def test_quarter_turn_exact(inter):
    # cos 0, sin 1: y_a = x_b, y_b = -x_a exactly; values past rot_dim untouched
    rng = np.random.default_rng(2)
    hd, rot = 48, 32
    x = _x(rng, 3, 2, hd)
    cs = np.concatenate([np.zeros((4, rot // 2)), np.ones((4, rot // 2))], 1).astype(np.float32)
    _, _, y = oracle.inv_rope_fp8(x, np.array([3, 1, 2], np.int32), cs, interleaved=inter)
    xv = bf16_bits_values(x).reshape(y.shape)
    for a, b in _pairs(hd, rot, inter):
        assert np.array_equal(y[..., a], xv[..., b])
        assert np.array_equal(y[..., b], -xv[..., a])
    assert np.array_equal(y[..., rot:], xv[..., rot:])


@pytest.mark.parametrize("hd,rot,inter", [(64, 64, 0), (128, 128, 1), (192, 64, 0), (80, 48, 1)])
def test_dense_rotation_matrix(hd, rot, inter):
    """y = R(p)^T x with R(p) the block rotation built from the table row of
    each token's position, applied as a float64 matrix product; the oracle's
    fp32 sums lie within 2 fp32 roundings of |x_a c| + |x_b s|."""
    rng = np.random.default_rng(hd + rot)
    T, nh, max_pos = 7, 4, 4096
    x = _x(rng, T, nh, hd, 3.0)
    pos = rng.integers(0, max_pos, T).astype(np.int32)
    cs = _table(max_pos, rot)
    _, _, y = oracle.inv_rope_fp8(x, pos, cs, interleaved=inter)
    xv = bf16_bits_values(x).reshape(T, nh, hd).astype(np.float64)
    half = rot // 2
    for t in range(T):
        R = np.eye(hd)
        mag = np.zeros(hd)
        for i, (a, b) in enumerate(_pairs(hd, rot, inter)):
            c, s = float(cs[pos[t], i]), float(cs[pos[t], half + i])
            R[a, a], R[a, b], R[b, a], R[b, b] = c, -s, s, c  # forward rotation
            mag[a] = mag[b] = 1.0
        want = xv[t] @ R  # row vectors: x R = (R^T x^T)^T, the inverse rotation
        bound = 2 * U * (np.abs(xv[t]) @ np.abs(R)) + 1e-300
        assert np.all(np.abs(y[t] - want) <= bound)
        # a rotation keeps each pair's length (to rounding)
        for a, b in _pairs(hd, rot, inter):
            n0 = xv[t][:, a] ** 2 + xv[t][:, b] ** 2
            n1 = y[t][:, a].astype(np.float64) ** 2 + y[t][:, b].astype(np.float64) ** 2
            assert np.all(np.abs(n1 - n0) <= 8 * U * n0 + 1e-30)


@pytest.mark.parametrize("hd,rot,inter", [(128, 128, 0), (64, 32, 1)])
def test_per_head_quantisation(hd, rot, inter):
    rng = np.random.default_rng(7)
    T, nh, max_pos = 9, 5, 512
    x = _x(rng, T, nh, hd, 2.0)
    x[2, 1, :] = 0  # a zero head
    pos = rng.integers(0, max_pos, T).astype(np.int32)
    cs = _table(max_pos, rot)
    codes, sc, y = oracle.inv_rope_fp8(x, pos, cs, interleaved=inter)
    # zero head: scale 1, every code +-0 (0 x a negative cosine is -0)
    assert sc[2, 1] == 1.0 and not (codes[2, 1] & 0x7F).any()
    dq = oracle.e4m3_decode(codes.ravel()).reshape(codes.shape) * sc[..., None].astype(np.float64)
    amax = np.max(np.abs(y.astype(np.float64)), axis=-1)
    for t in range(T):
        for h in range(nh):
            if amax[t, h] == 0:
                continue
            assert sc[t, h] == np.float32(np.float32(amax[t, h]) / np.float32(448.0))
            # the largest element takes the largest code magnitude
            j = int(np.argmax(np.abs(y[t, h])))
            assert codes[t, h, j] & 0x7F == 0x7E
            # dequantised codes within half an e4m3 step (relative 2^-4 for
            # normal codes, 2^-10 * scale below 2^-6) plus the fp32 rounding
            err = np.abs(dq[t, h] - y[t, h])
            assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(y[t, h]), 2.0 ** -10 * sc[t, h])
                          * (1 + 1e-6))


def test_positions_clamped_into_table():
    # positions beyond the table (a contract violation) read its last row
    rng = np.random.default_rng(3)
    x = _x(rng, 3, 2, 32)
    cs = _table(8, 32)
    a = oracle.inv_rope_fp8(x, np.array([7, 0, 7], np.int32), cs)
    b = oracle.inv_rope_fp8(x, np.array([100, -5, 8], np.int32), cs)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
