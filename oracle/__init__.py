"""CPU oracle for the fused Mixture-of-Experts layer -- TEST INFRASTRUCTURE.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding in ``moe_layer_gating_amd``) never imports it and shares no code
with it.

Two independent CPU references live here:

* ``moe_oracle.c`` (wrapped below): the plain per-token, per-selected-expert
  loop, accumulating in double.  It is built with gcc, no fast-math, with
  ``-ffp-contract=off`` so that every fp32 step (scales, x*r products) is a
  single IEEE operation.
* ``bruteforce.py``: a dense NumPy evaluation of every expert for every
  token, masked by the top-k choice, used to pin the oracle on tiny inputs.

Array conventions: bf16 tensors are NumPy ``uint16`` arrays of raw bits, FP8
e4m3 tensors are ``uint8`` codes, fp32 tensors are ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32, BF16, FP8 = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build of the same source, used
# when MOE_ORACLE_SANITIZE=1 (the process must preload the ASan runtime)
_LIB_SAN = os.path.join(_HERE, "libmoe_oracle_san.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
              "-fno-omit-frame-pointer", "-g"]
_lib = None


def _sanitized():
    return os.environ.get("MOE_ORACLE_SANITIZE") == "1"


def build(force: bool = True, sanitize: bool = False) -> str:
    """Compile the C oracle into ``oracle/libmoe_oracle.so`` (or, with
    ``sanitize``, the ASan/UBSan build ``oracle/libmoe_oracle_san.so``)."""
    lib = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(lib):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-Wall"] + (_SAN_FLAGS if sanitize else []) + ["-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, lib)
    return lib


def _load():
    global _lib
    if _lib is None:
        path = _LIB_SAN if _sanitized() else _LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(sanitize=_sanitized())
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_long
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode_array.argtypes = [P, i64, P]
        lib.oracle_e4m3_decode_array.argtypes = [P, i64, P]
        lib.oracle_bf16_round_array.argtypes = [P, i64, P]
        lib.oracle_router_logits.argtypes = [i32, i32, i32, i32, P, P, P]
        lib.oracle_topk_gating.argtypes = [P, i32, i32, i32, i32, P, P]
        lib.oracle_align_sort.argtypes = [P, i32, i32, i32, P, P, P, P]
        lib.oracle_act_quant.restype = ctypes.c_float
        lib.oracle_act_quant.argtypes = [P, i32, i64, P, P]
        lib.oracle_w13_swiglu.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, i64, P, P]
        lib.oracle_w2.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, i64, P, P]
        lib.oracle_combine.argtypes = [i32, i32, i32, i32, P, P, P, P, P]
        lib.oracle_combine_f32.argtypes = [i32, i32, i32, i32, P, P, P, P]
        lib.oracle_inv_rope_fp8.argtypes = [P, P, P] + [i32] * 6 + [P, P, P]
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [i32] * 7 + [P] * 16
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def act_dtype(mode):
    return np.float32 if mode == F32 else np.uint16


def w_dtype(mode):
    return {F32: np.float32, BF16: np.uint16, FP8: np.uint8}[mode]


# ---------------------------------------------------------------- codecs
def e4m3_encode(v):
    v = _c(v, np.float32).ravel()
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_decode(c):
    c = _c(c, np.uint8).ravel()
    out = np.empty(c.shape, np.float64)
    _load().oracle_e4m3_decode_array(_p(c), c.size, _p(out))
    return out


def bf16_round(v):
    """Round doubles to bf16 (RNE); returns the uint16 bit patterns."""
    v = _c(v, np.float64).ravel()
    out = np.empty(v.shape, np.uint16)
    _load().oracle_bf16_round_array(_p(v), v.size, _p(out))
    return out


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- steps
def router_logits(mode, x, wg):
    """logits[t][e] = sum_h x[t][h] * wg[e][h], summed exactly, rounded to fp32.
    x [T,H] and wg [E,H] in the activation type (fp32, or bf16 bits)."""
    x = _c(x, act_dtype(mode))
    wg = _c(wg, act_dtype(mode))
    T, H = x.shape
    E, H2 = wg.shape
    assert H2 == H
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits(mode, T, H, E, _p(x), _p(wg), _p(out))
    return out


def topk_gating(logits, k, renormalize=True):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().oracle_topk_gating(_p(logits), T, E, k, int(bool(renormalize)), _p(ids), _p(w))
    return ids, w


def align_sort(topk_ids, E):
    ids = _c(topk_ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_ids = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    _load().oracle_align_sort(_p(ids), T, k, E, _p(counts), _p(offsets), _p(sorted_ids), _p(inv))
    return counts, offsets, sorted_ids, inv


def act_quant(a, mode=BF16):
    """Per-tensor dynamic e4m3 quantisation: returns (codes, s, r)."""
    a = _c(a, act_dtype(mode))
    codes = np.empty(a.shape, np.uint8)
    r = ctypes.c_float(0.0)
    s = _load().oracle_act_quant(_p(a), mode, a.size, _p(codes), ctypes.byref(r))
    return codes, np.float32(s), np.float32(r.value)


def w13_swiglu(mode, x, w13, w13_scale, sorted_ids, offsets, k, positions=None):
    """h rows in sorted order ([T*k, I], activation dtype) and s_x.

    With ``positions`` only those rows are computed; the result then has
    ``len(positions)`` rows in that order.
    """
    x = _c(x, act_dtype(mode))
    w13 = _c(w13, w_dtype(mode))
    T, H = x.shape
    E, I2, H2 = w13.shape
    assert H2 == H
    I = I2 // 2
    sc = None if w13_scale is None else _c(w13_scale, np.float32)
    sorted_ids = _c(sorted_ids, np.int32)
    offsets = _c(offsets, np.int32)
    h = np.zeros((T * k, I), act_dtype(mode))
    s_x = ctypes.c_float(0.0)
    if positions is None:
        _load().oracle_w13_swiglu(mode, T, H, E, k, I, _p(x), _p(w13), _p(sc), _p(sorted_ids),
                                  _p(offsets), None, 0, _p(h), ctypes.byref(s_x))
        return h, np.float32(s_x.value)
    pos = _c(positions, np.int64).astype(np.int32)
    _load().oracle_w13_swiglu(mode, T, H, E, k, I, _p(x), _p(w13), _p(sc), _p(sorted_ids),
                              _p(offsets), _p(pos), pos.size, _p(h), ctypes.byref(s_x))
    return h[pos], np.float32(s_x.value)


def w2(mode, h, w2_, w2_scale, offsets, k, positions=None):
    """y (float64, rows = sorted positions or the listed positions) and s_h."""
    h = _c(h, act_dtype(mode))
    w2_ = _c(w2_, w_dtype(mode))
    E, H, I = w2_.shape
    n_pairs = h.shape[0]
    assert h.shape[1] == I and n_pairs % k == 0
    T = n_pairs // k
    sc = None if w2_scale is None else _c(w2_scale, np.float32)
    offsets = _c(offsets, np.int32)
    s_h = ctypes.c_float(0.0)
    if positions is None:
        y = np.empty((n_pairs, H), np.float64)
        _load().oracle_w2(mode, T, H, E, k, I, _p(h), _p(w2_), _p(sc), _p(offsets), None, 0, _p(y),
                          ctypes.byref(s_h))
    else:
        pos = _c(positions, np.int64).astype(np.int32)
        y = np.empty((pos.size, H), np.float64)
        _load().oracle_w2(mode, T, H, E, k, I, _p(h), _p(w2_), _p(sc), _p(offsets), _p(pos),
                          pos.size, _p(y), ctypes.byref(s_h))
    return y, np.float32(s_h.value)


def combine(mode, y, inv_perm, topk_weights, exact=False):
    """out[t] = sum_j w[t,j] * y[inv_perm[t*k+j]]; y float64 or float32.

    With ``exact`` (float64 y only) also returns the sums before their
    rounding to the output type: (out, out_exact)."""
    w = _c(topk_weights, np.float32)
    T, k = w.shape
    H = y.shape[1]
    inv = _c(inv_perm, np.int32)
    out = np.empty((T, H), act_dtype(mode))
    if y.dtype == np.float32:
        yy = _c(y, np.float32)
        _load().oracle_combine_f32(mode, T, H, k, _p(yy), _p(inv), _p(w), _p(out))
    else:
        yy = _c(y, np.float64)
        ex = np.empty((T, H), np.float64) if exact else None
        _load().oracle_combine(mode, T, H, k, _p(yy), _p(inv), _p(w), _p(out), _p(ex))
        if exact:
            return out, ex
    assert not exact, "exact sums need float64 y"
    return out


def forward(mode, x, logits, w13, w13_scale, w2_, w2_scale, k, renormalize=True):
    """The whole layer.  Returns a dict with out and every intermediate;
    ``out_exact`` holds out before its rounding to the output type."""
    x = _c(x, act_dtype(mode))
    logits = _c(logits, np.float32)
    w13 = _c(w13, w_dtype(mode))
    w2_ = _c(w2_, w_dtype(mode))
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    s13 = None if w13_scale is None else _c(w13_scale, np.float32)
    s2 = None if w2_scale is None else _c(w2_scale, np.float32)
    r = dict(
        out=np.empty((T, H), act_dtype(mode)),
        topk_ids=np.empty((T, k), np.int32),
        topk_weights=np.empty((T, k), np.float32),
        counts=np.empty(E, np.int32),
        offsets=np.empty(E + 1, np.int32),
        sorted_ids=np.empty(T * k, np.int32),
        inv_perm=np.empty(T * k, np.int32),
        h=np.empty((T * k, I), act_dtype(mode)),
        scales=np.empty(2, np.float32),
        out_exact=np.empty((T, H), np.float64),
    )
    rc = _load().oracle_forward(mode, T, H, E, k, I, int(bool(renormalize)), _p(x), _p(logits),
                                _p(w13), _p(s13), _p(w2_), _p(s2), _p(r["out"]), _p(r["topk_ids"]),
                                _p(r["topk_weights"]), _p(r["counts"]), _p(r["offsets"]),
                                _p(r["sorted_ids"]), _p(r["inv_perm"]), _p(r["h"]), _p(r["scales"]),
                                _p(r["out_exact"]))
    if rc != 0:
        raise MemoryError("oracle_forward: allocation failed")
    return r


def inv_rope_fp8(x, positions, cos_sin, rot_dim=None, interleaved=False):
    """Inverse rotary embedding then per-(token, head) e4m3 quantisation.

    x [T, n_heads, head_dim] bf16 bits (uint16); positions [T] int32;
    cos_sin [max_pos, rot_dim] fp32 (cosines, then sines, of the pair
    angles).  Returns (codes uint8 [T, n_heads, head_dim], scales fp32
    [T, n_heads], y fp32 [T, n_heads, head_dim] before quantisation)."""
    x = _c(x, np.uint16)
    T, nh, hd = x.shape
    cs = _c(cos_sin, np.float32)
    max_pos, rd = cs.shape
    assert rot_dim is None or rot_dim == rd
    pos = _c(positions, np.int32)
    assert pos.shape == (T,)
    codes = np.empty((T, nh, hd), np.uint8)
    scales = np.empty((T, nh), np.float32)
    y = np.empty((T, nh, hd), np.float32)
    _load().oracle_inv_rope_fp8(_p(x), _p(pos), _p(cs), T, nh, hd, rd, max_pos,
                                int(bool(interleaved)), _p(y), _p(codes), _p(scales))
    return codes, scales, y


def to_f64(a, mode):
    """Values of an activation array (fp32 or bf16 bits) as float64."""
    return np.asarray(a, np.float64) if mode == F32 else bf16_to_f64(a)
