"""Python binding of the fused MoE library for MI355X (gfx950).

Argument marshalling only: every function passes device pointers, sizes and
the current HIP stream to the C ABI declared in ``include/moe_gfx950.h`` and
raises ``MoeError`` on a non-zero status.  All computation happens in the HIP
kernels of ``libmoe_gfx950.so``; there is no fallback.  PyTorch provides the
device memory and the stream.

Tensor dtypes by mode (taken from the dtype of ``w13``):
  fp32 weights            -> fp32 mode: x, h, out fp32
  bf16 weights            -> bf16 mode: x, h, out bf16
  float8_e4m3fn or uint8  -> FP8 mode: e4m3 codes, fp32 scales [E]; x, h, out bf16
"""
from __future__ import annotations

import ctypes
import os

import torch

MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_gfx950.so")
_lib = None


class MoeError(RuntimeError):
    pass


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("wdtype", ctypes.c_int32),
                ("renormalize", ctypes.c_int32)]


class moe_routing_offsets(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in ("topk_ids", "topk_weights", "expert_counts",
                                                "expert_offsets", "sorted_ids", "inv_perm")]


EXPORTS = ("moe_check_shape", "moe_workspace_bytes", "moe_status_string",
           "moe_align_sort_workspace_bytes", "moe_workspace_routing", "moe_topk_gating",
           "moe_align_sort", "moe_grouped_gemm_w13_swiglu", "moe_grouped_gemm_w2", "moe_combine",
           "moe_act_quant_e4m3",
           "moe_fused_forward", "moe_fused_forward_events", "moe_router_logits",
           "moe_fused_forward_router", "moe_fused_forward_noalloc", "moe_inv_rope_fp8_quant")
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
# host-only calls whose return type is not a moe_status
_NON_STATUS = ("moe_workspace_bytes", "moe_status_string", "moe_align_sort_workspace_bytes")
NUM_STAGE_EVENTS = 9


def lib():
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError("libmoe_gfx950.so is not built; run __graft_entry__.build() "
                           "(or python moe_layer_gating_amd/_build.py)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        S = ctypes.POINTER(moe_shape)
        L.moe_check_shape.argtypes = [S]
        L.moe_check_shape.restype = ctypes.c_int
        L.moe_workspace_bytes.argtypes = [S]
        L.moe_workspace_bytes.restype = sz
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_align_sort_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_align_sort_workspace_bytes.restype = sz
        L.moe_workspace_routing.argtypes = [S, ctypes.POINTER(moe_routing_offsets)]
        L.moe_topk_gating.argtypes = [P, i32, i32, i32, i32, P, P, P]
        L.moe_align_sort.argtypes = [P, i32, i32, i32, P, P, P, P, P, sz, P]
        L.moe_grouped_gemm_w13_swiglu.argtypes = [S, P, P, P, P, P, P, P, P, sz, P]
        L.moe_grouped_gemm_w2.argtypes = [S, P, P, P, P, P, P, P, sz, P]
        L.moe_combine.argtypes = [S, P, P, P, P, P]
        L.moe_act_quant_e4m3.argtypes = [P, ctypes.c_int64, P, P, P]
        L.moe_fused_forward.argtypes = [S, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.moe_fused_forward_noalloc.argtypes = [S, P, P, P, P, P, P, P, P, P, P]
        L.moe_inv_rope_fp8_quant.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P, P]
        L.moe_router_logits.argtypes = [S, P, P, P, P, sz, P]
        L.moe_fused_forward_router.argtypes = [S, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        L.moe_fused_forward_events.argtypes = [S, P, P, P, P, P, P, P, P, P, P, sz, P,
                                               ctypes.POINTER(ctypes.c_void_p), i32]
        for name in EXPORTS:
            if name not in _NON_STATUS:
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc, what):
    if rc != 0:
        raise MoeError("%s failed: %d (%s)" % (what, rc, lib().moe_status_string(rc).decode()))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise MoeError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise MoeError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def mode_of(w):
    if w.dtype == torch.float32:
        return MOE_F32
    if w.dtype == torch.bfloat16:
        return MOE_BF16
    if w.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MOE_FP8_E4M3
    raise MoeError("unsupported weight dtype %s" % w.dtype)


def act_dtype(mode):
    return torch.float32 if mode == MOE_F32 else torch.bfloat16


def make_shape(T, H, E, k, I, mode, renormalize=True):
    return moe_shape(int(T), int(H), int(E), int(k), int(I), int(mode), int(bool(renormalize)))


def moe_check_shape(shape):
    return lib().moe_check_shape(ctypes.byref(shape))


def moe_workspace_bytes(shape):
    return lib().moe_workspace_bytes(ctypes.byref(shape))


def workspace(shape, device=None):
    """Allocate a workspace for `shape` (torch uint8, 256-byte aligned)."""
    n = moe_workspace_bytes(shape)
    if n == 0:
        raise MoeError("invalid shape")
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def moe_topk_gating(logits, k, renormalize=True, topk_ids=None, topk_weights=None):
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    _check(lib().moe_topk_gating(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(topk_ids),
                                 _ptr(topk_weights), _stream()), "moe_topk_gating")
    return topk_ids, topk_weights


def moe_align_sort_workspace_bytes(T, k, E):
    return lib().moe_align_sort_workspace_bytes(int(T), int(k), int(E))


def moe_align_sort(topk_ids, E, with_inv=True, ws=None):
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_ids = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev) if with_inv else None
    if ws is None:
        n = moe_align_sort_workspace_bytes(T, k, E)
        if n == 0:
            raise MoeError("invalid grouping shape T=%d k=%d E=%d" % (T, k, E))
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
    _check(lib().moe_align_sort(_ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets),
                                _ptr(sorted_ids), _ptr(inv), _ptr(ws), ws.numel(), _stream()),
           "moe_align_sort")
    return counts, offsets, sorted_ids, inv


def moe_workspace_routing(shape):
    """Byte offsets of the routing arrays the fused entry points leave in a
    workspace of `shape` (a moe_routing_offsets)."""
    r = moe_routing_offsets()
    _check(lib().moe_workspace_routing(ctypes.byref(shape), ctypes.byref(r)),
           "moe_workspace_routing")
    return r


def routing_from_workspace(ws, T, E, k, H=128, I=128, mode=MOE_BF16):
    """Views (no copies) of the grouping a fused call left in `ws`: counts
    [E], offsets [E+1], sorted_ids [T*k], inv_perm [T*k] (int32), plus the
    ids [T,k] and weights [T,k] slots (filled only when the call kept them in
    the workspace).  H, I and mode must be the call's when they change the
    workspace layout (they place only regions after these)."""
    r = moe_workspace_routing(make_shape(T, H, E, k, I, mode))

    def view(off, n, dt):
        return ws[off:off + 4 * n].view(dt)

    return dict(counts=view(r.expert_counts, E, torch.int32),
                offsets=view(r.expert_offsets, E + 1, torch.int32),
                sorted_ids=view(r.sorted_ids, T * k, torch.int32),
                inv_perm=view(r.inv_perm, T * k, torch.int32),
                topk_ids=view(r.topk_ids, T * k, torch.int32).view(T, k),
                topk_weights=view(r.topk_weights, T * k, torch.float32).view(T, k))


def moe_grouped_gemm_w13_swiglu(x, w13, w13_scale, sorted_ids, expert_offsets, k, ws=None, h=None,
                                act_scales=None):
    mode = mode_of(w13)
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    shape = make_shape(T, H, E, k, I, mode)
    ws = workspace(shape, x.device) if ws is None else ws
    if h is None:
        h = torch.empty((T * k, I), dtype=act_dtype(mode), device=x.device)
    if act_scales is None:
        act_scales = torch.zeros(4, dtype=torch.float32, device=x.device)
    _check(lib().moe_grouped_gemm_w13_swiglu(ctypes.byref(shape), _ptr(x), _ptr(w13),
                                             _ptr(w13_scale), _ptr(sorted_ids),
                                             _ptr(expert_offsets), _ptr(h), _ptr(act_scales),
                                             _ptr(ws), ws.numel(), _stream()),
           "moe_grouped_gemm_w13_swiglu")
    return h, act_scales


def moe_grouped_gemm_w2(h, w2, w2_scale, expert_offsets, act_scales, k, ws=None, y=None):
    mode = mode_of(w2)
    n_pairs, I = h.shape
    E, H, _ = w2.shape
    T = n_pairs // k
    shape = make_shape(T, H, E, k, I, mode)
    ws = workspace(shape, h.device) if ws is None else ws
    if y is None:
        y = torch.empty((n_pairs, H), dtype=torch.float32, device=h.device)
    _check(lib().moe_grouped_gemm_w2(ctypes.byref(shape), _ptr(h), _ptr(w2), _ptr(w2_scale),
                                     _ptr(expert_offsets), _ptr(act_scales), _ptr(y), _ptr(ws),
                                     ws.numel(), _stream()), "moe_grouped_gemm_w2")
    return y


def moe_act_quant_e4m3(a, codes=None, scales=None):
    """Per-tensor e4m3 codes of a bf16 tensor: (codes uint8, scales [s, amax] fp32)."""
    n = a.numel()
    if codes is None:
        codes = torch.empty(a.shape, dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty(2, dtype=torch.float32, device=a.device)
    _check(lib().moe_act_quant_e4m3(_ptr(a), n, _ptr(codes), _ptr(scales), _stream()),
           "moe_act_quant_e4m3")
    return codes, scales


def moe_combine(y, inv_perm, topk_weights, mode, E=None, I=128, out=None):
    T, k = topk_weights.shape
    H = y.shape[1]
    shape = make_shape(T, H, E or k, k, I, mode)
    if out is None:
        out = torch.empty((T, H), dtype=act_dtype(mode), device=y.device)
    _check(lib().moe_combine(ctypes.byref(shape), _ptr(y), _ptr(inv_perm), _ptr(topk_weights),
                             _ptr(out), _stream()), "moe_combine")
    return out


def moe_fused_forward(x, logits, w13, w13_scale, w2, w2_scale, k, renormalize=True, out=None,
                      ws=None, topk_ids=None, topk_weights=None):
    mode = mode_of(w13)
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    shape = make_shape(T, H, E, k, I, mode, renormalize)
    ws = workspace(shape, x.device) if ws is None else ws
    if out is None:
        out = torch.empty((T, H), dtype=act_dtype(mode), device=x.device)
    _check(lib().moe_fused_forward(ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w13),
                                   _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(out),
                                   _ptr(topk_ids), _ptr(topk_weights), _ptr(ws), ws.numel(),
                                   _stream()), "moe_fused_forward")
    return out


def moe_fused_forward_noalloc(x, logits, w13, w13_scale, w2, w2_scale, k, out,
                              renormalize=True, topk_ids=None, topk_weights=None):
    """moe_fused_forward on the library's static scratch: no workspace, and
    the caller passes `out` (nothing is allocated here either)."""
    mode = mode_of(w13)
    T, H = x.shape
    E, I2, _ = w13.shape
    shape = make_shape(T, H, E, k, I2 // 2, mode, renormalize)
    _check(lib().moe_fused_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w13),
                                           _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(out),
                                           _ptr(topk_ids), _ptr(topk_weights), _stream()),
           "moe_fused_forward_noalloc")
    return out


def moe_inv_rope_fp8_quant(x, positions, cos_sin, interleaved=False, codes=None, scales=None):
    """Inverse rotary embedding + per-(token, head) e4m3 quantisation.
    x [T, n_heads, head_dim] bf16, positions [T] int32, cos_sin [max_pos,
    rot_dim] fp32 -> (codes uint8 [T, n_heads, head_dim], scales fp32
    [T, n_heads])."""
    T, nh, hd = x.shape
    max_pos, rot = cos_sin.shape
    if codes is None:
        codes = torch.empty((T, nh, hd), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((T, nh), dtype=torch.float32, device=x.device)
    _check(lib().moe_inv_rope_fp8_quant(_ptr(x), _ptr(positions), _ptr(cos_sin), T, nh, hd, rot,
                                        max_pos, int(bool(interleaved)), _ptr(codes),
                                        _ptr(scales), _stream()), "moe_inv_rope_fp8_quant")
    return codes, scales


def moe_router_logits(x, wg, E=None, k=1, ws=None, logits=None):
    """Router GEMM: logits [T,E] fp32 = x [T,H] . wg [E,H]^T (fp32 or bf16
    operands of the same type, fp32 accumulation)."""
    T, H = x.shape
    E_, H2 = wg.shape
    assert H2 == H and (E is None or E == E_)
    mode = MOE_F32 if x.dtype == torch.float32 else MOE_BF16
    # the workspace depends only on T, H, E here; a minimal expert FFN shape
    shape = make_shape(T, H, E_, min(k, E_), 128, mode)
    ws = workspace(shape, x.device) if ws is None else ws
    if logits is None:
        logits = torch.empty((T, E_), dtype=torch.float32, device=x.device)
    _check(lib().moe_router_logits(ctypes.byref(shape), _ptr(x), _ptr(wg), _ptr(logits), _ptr(ws),
                                   ws.numel(), _stream()), "moe_router_logits")
    return logits


def moe_fused_forward_router(x, wg, w13, w13_scale, w2, w2_scale, k, renormalize=True, out=None,
                             ws=None, logits=None, topk_ids=None, topk_weights=None):
    """The whole layer from x and the router weights wg [E,H] (activation
    type); `logits` (optional [T,E] fp32) receives the router output."""
    mode = mode_of(w13)
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    assert tuple(wg.shape) == (E, H) and wg.dtype == act_dtype(mode)
    shape = make_shape(T, H, E, k, I, mode, renormalize)
    ws = workspace(shape, x.device) if ws is None else ws
    if out is None:
        out = torch.empty((T, H), dtype=act_dtype(mode), device=x.device)
    _check(lib().moe_fused_forward_router(ctypes.byref(shape), _ptr(x), _ptr(wg), _ptr(w13),
                                          _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(out),
                                          _ptr(logits), _ptr(topk_ids), _ptr(topk_weights),
                                          _ptr(ws), ws.numel(), _stream()),
           "moe_fused_forward_router")
    return out


def moe_fused_forward_events(x, logits, w13, w13_scale, w2, w2_scale, k, events, renormalize=True,
                             out=None, ws=None, topk_ids=None, topk_weights=None):
    """moe_fused_forward that also records the given hipEvent_t handles
    (NUM_STAGE_EVENTS integers, 0 or None to skip a boundary) at the stage
    boundaries."""
    mode = mode_of(w13)
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    shape = make_shape(T, H, E, k, I, mode, renormalize)
    ws = workspace(shape, x.device) if ws is None else ws
    if out is None:
        out = torch.empty((T, H), dtype=act_dtype(mode), device=x.device)
    ev = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e or None) for e in events])
    _check(lib().moe_fused_forward_events(ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w13),
                                          _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(out),
                                          _ptr(topk_ids), _ptr(topk_weights), _ptr(ws), ws.numel(),
                                          _stream(), ev, len(events)), "moe_fused_forward_events")
    return out
