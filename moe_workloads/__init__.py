"""Seeded synthetic inputs for the fused MoE layer.

This module only draws random numbers and converts them to the storage types
of the layer's inputs.  It holds none of the layer's own arithmetic; both the
GPU tests and the CPU oracle consume what it returns.

Recipe (all draws from ``numpy.random.SeedSequence(seed)``; children spawned
in this fixed order: x, Wg, routing extras, expert weights; the weight child
spawns 2E grandchildren, w13[e] then w2[e]):

* x ~ N(0, 1) drawn in fp32; bf16 layers round it to bf16 (PyTorch cast, RNE).
* router logits = x . Wg with Wg ~ N(0, 0.02), accumulated in float64 from the
  (rounded) x and rounded once to fp32.  The router product is input
  preparation: the layer starts from the logits.
* expert weights ~ N(0, 0.02).  bf16 layers round them with PyTorch.  FP8
  layers quantise each expert's w13 and w2 separately: amax over the matrix,
  scale = amax / 448 (fp32), codes = e4m3(clamp(w * 448 / amax, +-448)) with
  PyTorch's ``float8_e4m3fn`` cast (round to nearest even).
* "zipf" routing adds b_e = -1.1 * ln(r_e) to the logits, r a seeded
  permutation of 1..E, which skews the expert load like a Zipf(1.1) law.
* "empty" routing sets the logits of round(0.1 * E) seeded experts to -inf,
  so those experts receive no tokens.
* the decode FP8 layer uses one weight set for T = 1, 4 and 16; x and the
  logits are the first T rows of one 16-row draw.

Storage: bf16 arrays are ``uint16`` bit patterns, FP8 arrays ``uint8`` codes,
fp32 arrays ``float32``.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import os

import numpy as np
import torch

F32, BF16, FP8 = 0, 1, 2
MODE_NAMES = {F32: "f32", BF16: "bf16", FP8: "fp8"}


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    mode: int
    routing: str = "uniform"  # "uniform" | "zipf" | "empty"
    draw_T: int = 0  # rows drawn for x/logits (0 = T); decode FP8 draws 16 and keeps T
    seed: int = 0


# The five layer shapes the path is built for, plus the prefill dims in the
# compute-bound regime.
WORKLOADS = {
    "tiny_f32": LayerSpec("tiny_f32", 16, 128, 8, 2, 256, F32),
    "decode_bf16": LayerSpec("decode_bf16", 8, 4096, 8, 2, 14336, BF16),
    "decode_fp8_t1": LayerSpec("decode_fp8_t1", 1, 4096, 64, 8, 8192, FP8, draw_T=16),
    "decode_fp8_t4": LayerSpec("decode_fp8_t4", 4, 4096, 64, 8, 8192, FP8, draw_T=16),
    "decode_fp8_t16": LayerSpec("decode_fp8_t16", 16, 4096, 64, 8, 8192, FP8, draw_T=16),
    "prefill_fp8": LayerSpec("prefill_fp8", 4096, 7168, 256, 8, 2048, FP8, routing="zipf"),
    "mixed_fp8": LayerSpec("mixed_fp8", 512, 6144, 128, 8, 4096, FP8, routing="empty"),
    # the prefill layer's dims at four times the tokens (mean 512 pairs per
    # expert): the compute-bound regime, an extra labelled measurement
    "prefill_fp8_t16k": LayerSpec("prefill_fp8_t16k", 16384, 7168, 256, 8, 2048, FP8,
                                  routing="zipf"),
}


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal(ss, shape, std):
    g = np.random.Generator(np.random.PCG64(ss))
    a = g.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def to_bf16_bits(a32):
    t = torch.from_numpy(np.ascontiguousarray(a32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_values(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fp8_quantise_matrix(w32):
    """Per-matrix weight quantisation for input preparation (PyTorch cast)."""
    t = torch.from_numpy(w32)
    amax = float(t.abs().max())
    if amax == 0.0:
        return np.zeros(w32.shape, np.uint8), np.float32(1.0)
    scale = np.float32(np.float32(amax) / np.float32(448.0))
    r = np.float32(np.float32(448.0) / np.float32(amax))
    q = (t * float(r)).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), scale


def _weights_for_expert(ss13, ss2, H, I, mode):
    w13 = _normal(ss13, (2 * I, H), 0.02)
    w2 = _normal(ss2, (H, I), 0.02)
    if mode == F32:
        return w13, None, w2, None
    if mode == BF16:
        return to_bf16_bits(w13), None, to_bf16_bits(w2), None
    q13, s13 = _fp8_quantise_matrix(w13)
    q2, s2 = _fp8_quantise_matrix(w2)
    return q13, s13, q2, s2


def make_layer(spec: LayerSpec, with_weights: bool = True):
    """Draw one layer.  Returns a dict of NumPy arrays plus the spec."""
    T, H, E, k, I, mode = spec.T, spec.H, spec.E, spec.k, spec.I, spec.mode
    root = np.random.SeedSequence(spec.seed)
    ss_x, ss_wg, ss_route, ss_w = root.spawn(4)
    dT = spec.draw_T or T
    x32 = _normal(ss_x, (dT, H), 1.0)[:T]
    if mode == F32:
        x = np.ascontiguousarray(x32)
        xv = x.astype(np.float64)
    else:
        x = to_bf16_bits(x32)
        xv = bf16_bits_values(x).astype(np.float64)
    wg = _normal(ss_wg, (H, E), 0.02).astype(np.float64)
    logits64 = xv @ wg
    if spec.routing == "zipf":
        g = np.random.Generator(np.random.PCG64(ss_route))
        ranks = g.permutation(E) + 1
        logits64 = logits64 + (-1.1 * np.log(ranks.astype(np.float64)))[None, :]
    logits = logits64.astype(np.float32)
    if spec.routing == "empty":
        g = np.random.Generator(np.random.PCG64(ss_route))
        n_empty = int(round(0.1 * E))
        empty = np.sort(g.choice(E, size=n_empty, replace=False))
        logits[:, empty] = -np.inf
    # the router weights as a router GEMM consumes them: one row per expert,
    # in the activation type (the logits above use the unrounded draw)
    wg_rows = np.ascontiguousarray(wg.T.astype(np.float32))
    wg_act = wg_rows if mode == F32 else to_bf16_bits(wg_rows)
    layer = dict(spec=spec, x=x, logits=np.ascontiguousarray(logits), wg=wg_act)
    if with_weights:
        kids = ss_w.spawn(2 * E)
        wdt = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}[mode]
        w13 = np.empty((E, 2 * I, H), wdt)
        w2 = np.empty((E, H, I), wdt)
        s13 = np.ones(E, np.float32)
        s2 = np.ones(E, np.float32)

        def one(e):
            a, sa, b, sb = _weights_for_expert(kids[e], kids[E + e], H, I, mode)
            w13[e] = a
            w2[e] = b
            if sa is not None:
                s13[e] = sa
                s2[e] = sb

        with cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(one, range(E)))
        layer.update(w13=w13, w2=w2)
        layer.update(w13_scale=s13 if mode == FP8 else None, w2_scale=s2 if mode == FP8 else None)
    return layer


def planted_logits(T, E, k, counts, seed=0):
    """Router logits whose top-k choice hands expert e exactly counts[e] of
    the T*k pairs (sum(counts) == T*k, every count <= T).

    The pairs are listed expert by expert and pair i goes to token i % T, so
    a token's k experts are distinct (an expert's run of <= T pairs never
    wraps onto the same token twice).  A token's j-th planted expert gets a
    logit near 8 - 2j; every other logit is drawn from N(0, 0.5^2) clipped
    below 2, so the planted experts are the top k in their planted order.
    """
    counts = np.asarray(counts, np.int64)
    assert counts.size == E and counts.sum() == T * k and counts.max(initial=0) <= T
    g = np.random.default_rng(seed)
    logits = np.minimum(g.normal(0.0, 0.5, (T, E)), 2.0)
    experts = np.repeat(np.arange(E), counts)
    for i, e in enumerate(experts):
        t, j = i % T, i // T
        logits[t, e] = 8.0 - 2.0 * j + 0.1 * g.random()
    return np.ascontiguousarray(logits.astype(np.float32))


def scaled(name, T, H, E, k, I, mode, routing="uniform", seed=0):
    """A layer of arbitrary shape drawn with the same recipe."""
    return LayerSpec(name, T, H, E, k, I, mode, routing=routing, seed=seed)


# --------------------------------------------------------------------------
# Inputs of the inverse rotary embedding + per-head FP8 quantisation step.
# x ~ N(0, 1) drawn in fp32 and rounded to bf16; positions: a prefill batch
# takes consecutive positions from a seeded start, a decode batch one seeded
# position per token; the cos/sin table holds, per position p and pair i,
# cos(p * base^(-2i/rot_dim)) then sin(...), evaluated in float64 and rounded
# once to fp32 (base 10000, the usual rotary schedule).  The table is an
# input of the step, like the router logits of the layer.
@dataclasses.dataclass(frozen=True)
class RopeSpec:
    name: str
    T: int
    n_heads: int
    head_dim: int
    rot_dim: int
    max_pos: int
    interleaved: bool = False
    positions: str = "prefill"  # "prefill" | "random"
    seed: int = 0


ROPE_WORKLOADS = {
    # a 4096-token prefill batch, 32 heads of 128 values rotated in full
    "rope_prefill": RopeSpec("rope_prefill", 4096, 32, 128, 128, 8192),
    # a 16-token decode batch at scattered positions
    "rope_decode": RopeSpec("rope_decode", 16, 32, 128, 128, 8192, positions="random"),
}


def rope_table(max_pos, rot_dim, base=10000.0):
    half = rot_dim // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / rot_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * theta[None, :]
    return np.ascontiguousarray(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32))


def make_rope(spec: RopeSpec):
    root = np.random.SeedSequence(spec.seed)
    ss_x, ss_p = root.spawn(2)
    x32 = _normal(ss_x, (spec.T, spec.n_heads, spec.head_dim), 1.0)
    x = to_bf16_bits(x32.reshape(spec.T, -1)).reshape(x32.shape)
    g = np.random.Generator(np.random.PCG64(ss_p))
    if spec.positions == "prefill":
        start = int(g.integers(0, max(1, spec.max_pos - spec.T + 1)))
        pos = np.arange(start, start + spec.T) % spec.max_pos
    else:
        pos = g.integers(0, spec.max_pos, spec.T)
    return dict(spec=spec, x=np.ascontiguousarray(x), positions=pos.astype(np.int32),
                cos_sin=rope_table(spec.max_pos, spec.rot_dim))


def scaled_rope(name, T, n_heads, head_dim, rot_dim, max_pos, interleaved=False,
                positions="random", seed=0):
    return RopeSpec(name, T, n_heads, head_dim, rot_dim, max_pos, interleaved, positions, seed)
