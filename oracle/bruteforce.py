"""Dense brute-force evaluation of the MoE layer -- TEST INFRASTRUCTURE.

Used only to pin the C oracle on tiny inputs.  It is written independently of
``moe_oracle.c``: every expert is evaluated for every token in float64 with
NumPy matrix products, and the top-k choice is applied afterwards as a mask.
Routing uses a library stable sort, rounding uses PyTorch's dtype casts
(``torch.bfloat16`` and ``torch.float8_e4m3fn``, which round to nearest even;
the FP8 cast is preceded by a clamp to +-448 because PyTorch maps
out-of-range values to NaN rather than saturating).

Modes: 0 = fp32, 1 = bf16, 2 = FP8 e4m3 weights with bf16 activations.
"""
from __future__ import annotations

import numpy as np
import torch

F32, BF16, FP8 = 0, 1, 2


def bf16_bits_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def f64_to_bf16_values(v):
    """Round to bf16 with PyTorch and return the values as float64."""
    return torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def e4m3_codes_to_f64(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def f32_to_e4m3_values(v32):
    """Nearest-even e4m3 value of fp32 inputs with saturation, as float64."""
    t = torch.from_numpy(np.asarray(v32, np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def _act_values(a, mode):
    return np.asarray(a, np.float64) if mode == F32 else bf16_bits_to_f64(a)


def _w_values(w, mode):
    if mode == F32:
        return np.asarray(w, np.float64)
    if mode == BF16:
        return bf16_bits_to_f64(w)
    return e4m3_codes_to_f64(w)


def _quantise_dense(vals64):
    """Per-tensor dynamic quantisation of bf16 values: (decoded codes, s)."""
    A = np.float32(np.max(np.abs(vals64))) if vals64.size else np.float32(0)
    if A > 0:
        s = np.float32(A) / np.float32(448.0)
        r = np.float32(448.0) / np.float32(A)
    else:
        s = r = np.float32(1.0)
    prod = (vals64.astype(np.float32) * r).astype(np.float32)
    return f32_to_e4m3_values(prod), s


def routing(logits, k, renormalize=True):
    """Top-k by a stable library sort; weights from the full float64 softmax."""
    l = np.asarray(logits, np.float64)
    order = np.argsort(-l, axis=1, kind="stable")
    ids = order[:, :k]
    m = np.max(l, axis=1, keepdims=True)
    p = np.exp(l - m)
    p = p / p.sum(axis=1, keepdims=True)
    psel = np.take_along_axis(p, ids, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True) if renormalize else psel
    return ids.astype(np.int32), w


def grouping(ids, E):
    flat = np.asarray(ids).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    sorted_ids = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(sorted_ids)
    inv[sorted_ids] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_ids, inv


def forward(mode, x, logits, w13, w13_scale, w2, w2_scale, k, renormalize=True):
    """Dense evaluation; returns out (float64 values after the output rounding)."""
    xa = _act_values(x, mode)
    T, H = xa.shape
    W13 = _w_values(w13, mode)
    W2 = _w_values(w2, mode)
    E, I2, _ = W13.shape
    I = I2 // 2
    ids, gw = routing(logits, k, renormalize)
    mask = np.zeros((T, E), bool)
    gate = np.zeros((T, E), np.float64)
    for j in range(k):
        mask[np.arange(T), ids[:, j]] = True
        gate[np.arange(T), ids[:, j]] = gw[:, j]

    if mode == FP8:
        xq, s_x = _quantise_dense(xa)
        xin = xq
        c13 = (np.float32(s_x) * np.asarray(w13_scale, np.float32)).astype(np.float64)
    else:
        xin = xa
        c13 = np.ones(E)
    # every expert for every token: [T, E, 2I]
    Z = np.einsum("th,enh->ten", xin, W13) * c13[None, :, None]
    G, U = Z[..., :I], Z[..., I:]
    Hd = G / (1.0 + np.exp(-G)) * U
    if mode == F32:
        Hd = Hd.astype(np.float32).astype(np.float64)
    else:
        Hd = f64_to_bf16_values(Hd)
    if mode == FP8:
        routed = Hd[mask]  # [T*k, I]: the quantisation scale uses routed pairs only
        A = np.float32(np.max(np.abs(routed))) if routed.size else np.float32(0)
        if A > 0:
            s_h = np.float32(A) / np.float32(448.0)
            r_h = np.float32(448.0) / np.float32(A)
        else:
            s_h = r_h = np.float32(1.0)
        Hin = f32_to_e4m3_values((Hd.astype(np.float32) * r_h).astype(np.float32))
        c2 = (np.float32(s_h) * np.asarray(w2_scale, np.float32)).astype(np.float64)
    else:
        Hin = Hd
        c2 = np.ones(E)
    Y = np.einsum("ten,emn->tem", Hin, W2) * c2[None, :, None]
    out = np.einsum("te,tem->tm", gate * mask, Y)
    if mode == F32:
        return out.astype(np.float32).astype(np.float64)
    return f64_to_bf16_values(out)
