#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

One step = one call of moe_fused_forward over one batch: gating, grouping,
(FP8: activation quantisation), gate/up GEMM + SwiGLU, (FP8: h quantisation),
down GEMM and the weighted combine, with every input already resident in HBM.

Default workload: the prefill FP8 layer (4096 tokens, hidden 7168, 256
experts, top-8, SwiGLU intermediate 2048, e4m3 weights with per-expert
scales, Zipf(1.1)-skewed routing), the largest single-GPU layer of the
metric, whose prefill half is quoted in MFMA TFLOP/s.  The bf16 decode layer
(8 tokens, hidden 4096, 8 experts, top-2, intermediate 14336) is measured in
the same run as a labelled sub-record (`sub_records`).  Other layers:
--workload decode_bf16 | decode_fp8_t1 | decode_fp8_t4 | decode_fp8_t16 |
mixed_fp8 | prefill_fp8_t16k (the prefill dims at 16384 tokens,
compute-bound) | tiny_f32; --sub takes a comma list of sub-record layers, or
"none".  Inputs are seeded synthetic tensors (moe_workloads).

Prints ONE JSON line with tokens/s as `value`, plus:
  layer_hbm_frac / layer_mfma_frac -- the layer's algorithmic bytes and flops
                  per step against 8 TB/s and against the dense MFMA peak of
                  the layer's arithmetic type (FP8 layers: 5.0 PFLOP/s for
                  every flop); layer_mfma_frac_issued prices each GEMM at the
                  peak of the MFMA type its kernel issues (the few-token FP8
                  gate/up on the bf16 MFMA, 2.5 PFLOP/s), a secondary figure;
  roofline     -- the dominant kernel (the gate/up GEMM): its algorithmic
                  bytes (or flops) per launch / its average duration, timed
                  with HIP events taken by that kernel's own dispatch in
                  each of K further steps right after the timed ones
                  (ms_per_step_kernel_timed is their wall time per step),
                  against 8 TB/s (or the MFMA
                  peak of the layer's type when its arithmetic intensity is
                  above that ridge); `traffic` = its HBM bytes per launch from
                  rocprofv3 FETCH_SIZE / WRITE_SIZE counters
                  (profiles/traffic.json), null when the kernel sources have
                  changed since those counters were taken;
  cpu_baseline -- the CPU oracle timed on this host on a bounded sample of
                  the same workload (whole layers for the few-token layers;
                  the first tokens of the batch, full weights, for the
                  many-token ones), about 10 s;
  graph_replay -- the same step replayed from a captured HIP graph, as a
                  separate figure;
  flushed      -- single calls timed alone (event pair around each call) after
                  reading a 1 GiB buffer that evicts L2 and the 256 MB MALL:
                  median, p10 and p90 over 100 calls (few-token layers) or 20
                  (tiled layers), as a separate figure;
  router       -- the layer run from the router weights instead of the logits
                  (moe_fused_forward_router: for few-token bf16/FP8 batches
                  the front kernel computes the logits itself, one launch
                  fewer), per step, and the router GEMM alone, as separate
                  figures (also in each sub-record);
  sub_records  -- the same step figures for the sub-record layers; for
                  rope_prefill / rope_decode, the inverse rotary embedding +
                  per-head FP8 quantisation step (moe_inv_rope_fp8_quant):
                  its launch time and bytes against 8 TB/s.
"""
from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# dense MFMA peak of the layer's arithmetic type (fp32, bf16, FP8 e4m3)
MFMA_PEAK_TFLOPS = {0: 157.3, 1: 2500.0, 2: 5000.0}


def issued_mfma(mode, big):
    """MFMA type and dense peak (TFLOP/s) each GEMM's kernel issues, as
    ((gate/up type, peak), (down type, peak)).  FP8 layers: the tiled
    (many-token) kernels use the FP8 MFMA for both projections; the
    few-token kernels widen the gate/up codes to bf16 and use the bf16 MFMA
    (as fast there, where weights stream from HBM), the FP8 MFMA for the
    down projection."""
    if mode == 2:
        return (("fp8e4m3", 5000.0) if big else ("bf16 (e4m3 codes widened)", 2500.0),
                ("fp8e4m3", 5000.0))
    return ((DTYPE_NAME[mode], MFMA_PEAK_TFLOPS[mode]),) * 2

METRIC = "fused-MoE layer tokens/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)"
DTYPE_NAME = {0: "f32", 1: "bf16", 2: "fp8e4m3"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "moe_layer_gating_amd", "csrc")


def log(*a):
    print("bench:", *a, file=sys.stderr, flush=True)


def hip():
    h = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded
    h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    h.hipEventDestroy.argtypes = [ctypes.c_void_p]
    h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return h


def kernel_sources(big):
    """Source files that define the dominant kernel of a shape class."""
    names = ["gemm_tiles.hip" if big else "gemm_skinny.hip", "moe_common.h"]
    return [os.path.join(CSRC, n) for n in names]


ROPE_SOURCES = [os.path.join(CSRC, n) for n in ("rope.hip", "moe_common.h")]


def sources_sha256(files):
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_for(workload, kernel, files):
    """HBM bytes per launch of the dominant kernel from the stored counter
    runs, or None if there are none or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel") != kernel:
        return None
    if rec.get("sources_sha256") != sources_sha256(files):
        return None
    return (rec["fetch_kib"] * rec["fetch_scale"] + rec["write_kib"] * rec["write_scale"]) * 1024


def algorithmic(spec, counts):
    """Bytes / flops the method must move / compute (padding excluded)."""
    T, H, E, k, I, mode = spec.T, spec.H, spec.E, spec.k, spec.I, spec.mode
    bw = {0: 4, 1: 2, 2: 1}[mode]
    bx = 4 if mode == 0 else 2
    active = int((counts > 0).sum())
    scale_b = 8 * active if mode == 2 else 0
    layer_bytes = active * 3 * H * I * bw + scale_b + T * H * bx + 4 * T * E + T * H * bx
    flops = 6.0 * T * k * H * I
    # gate/up kernel: the active experts' w13 rows (+ FP8 scales), the token
    # rows it reads (e4m3 codes in FP8 mode) and the h it writes
    w13_bytes = active * 2 * I * H * bw + (4 * active if mode == 2 else 0) + T * H * (
        1 if mode == 2 else bx) + T * k * I * bx
    w13_flops = 4.0 * T * k * H * I
    return active, layer_bytes, flops, w13_bytes, w13_flops


def cpu_baseline(L, budget_s=10.0):
    """Time the CPU oracle on this workload for about budget_s: whole layers,
    repeated, when one layer takes a fraction of the budget; otherwise one
    run on the first tokens of the batch (all weights, all k experts of each
    token), sized from a 16-token calibration run."""
    import oracle

    s = L["spec"]
    threads = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    cores = min(int(omp) if omp and omp.isdigit() else threads, threads)

    def run(n_tok):
        t0 = time.perf_counter()
        oracle.forward(s.mode, L["x"][:n_tok], L["logits"][:n_tok], L["w13"], L["w13_scale"],
                       L["w2"], L["w2_scale"], s.k)
        return time.perf_counter() - t0

    n_cal = min(s.T, 16)
    t_cal = run(n_cal)
    if n_cal == s.T and t_cal < budget_s:  # whole layers, repeated
        n, el = 1, t_cal
        while el < budget_s and el / n * (n + 1) <= 3 * budget_s:
            el += run(s.T)
            n += 1
        return dict(value=s.T * n / el, unit="tokens/s", cores=cores, kind="oracle",
                    sample="%d full layer forward(s) of %s (%d tokens each), %.1f s" % (
                        n, s.name, s.T, el))
    n_tok = max(n_cal, min(s.T, int(n_cal * budget_s / max(t_cal, 1e-3))))
    el = run(n_tok) if n_tok != n_cal else t_cal
    return dict(value=n_tok / el, unit="tokens/s", cores=cores, kind="oracle",
                sample="first %d of the %d tokens of %s (full weights, every routed expert of "
                       "each token: gating through aggregation), one forward, %.1f s" % (
                           n_tok, s.T, s.name, el))


class Layer:
    """One seeded workload uploaded to the GPU, with its workspace."""

    def __init__(self, name):
        import numpy as np
        import torch

        import moe_layer_gating_amd as moe
        import moe_workloads as wl

        self.spec = spec = wl.WORKLOADS[name]
        log("generating", spec.name)
        self.L = L = wl.make_layer(spec)
        mode = spec.mode

        def dev_act(a):
            if mode == 0:
                return torch.from_numpy(a).cuda()
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()

        def dev_w(w):
            if mode == 0:
                return torch.from_numpy(w).cuda()
            if mode == 1:
                return torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).cuda()
            return torch.from_numpy(w).cuda()

        self.x = dev_act(L["x"])
        self.logits = torch.from_numpy(L["logits"]).cuda()
        self.w13 = dev_w(L["w13"])
        self.w2 = dev_w(L["w2"])
        self.wg = dev_act(L["wg"])
        self.s13 = None if L["w13_scale"] is None else torch.from_numpy(L["w13_scale"]).cuda()
        self.s2 = None if L["w2_scale"] is None else torch.from_numpy(L["w2_scale"]).cuda()
        shape = moe.make_shape(spec.T, spec.H, spec.E, spec.k, spec.I, mode)
        self.ws = moe.workspace(shape)
        self.out = torch.empty((spec.T, spec.H), dtype=moe.act_dtype(mode), device="cuda")
        self.ids = torch.empty((spec.T, spec.k), dtype=torch.int32, device="cuda")
        self.big = mode != 0 and spec.T * spec.k >= 16 * spec.E  # the tiled shape class
        self.kernel = "w13_swiglu_tiles" if self.big else "w13_swiglu_skinny"

    def step(self, events=None):
        import moe_layer_gating_amd as moe

        s = self.spec
        if events is None:
            moe.moe_fused_forward(self.x, self.logits, self.w13, self.s13, self.w2, self.s2, s.k,
                                  out=self.out, ws=self.ws, topk_ids=self.ids)
        else:
            moe.moe_fused_forward_events(self.x, self.logits, self.w13, self.s13, self.w2,
                                         self.s2, s.k, events, out=self.out, ws=self.ws,
                                         topk_ids=self.ids)


def measure(name, args, H_, full):
    """Time `args.steps` steps of one workload; with `full` also the separate
    figures (graph replay, router, flushed calls, stage breakdown, CPU
    baseline).  Returns the workload's record."""
    import numpy as np
    import torch

    import moe_layer_gating_amd as moe

    lay = Layer(name)
    spec, mode = lay.spec, lay.spec.mode

    def new_event():
        e = ctypes.c_void_p()
        assert H_.hipEventCreate(ctypes.byref(e)) == 0
        return e.value

    def elapsed_ms(a, b):
        f = ctypes.c_float()
        assert H_.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return f.value

    log("%s: warmup %d" % (name, args.warmup))
    for _ in range(args.warmup):
        lay.step()
    torch.cuda.synchronize()
    counts = np.bincount(lay.ids.cpu().numpy().ravel(), minlength=spec.E)

    # timed region: K plain steps (moe_fused_forward, as a caller runs it)
    log("%s: timing %d steps" % (name, args.steps))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        lay.step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # the dominant kernel's duration: K more steps, each taking the gate/up
    # GEMM dispatch's own start / end time (stage boundaries 4 and 5, on the
    # stream the kernels run on); that instrumentation adds host work per
    # step, so these steps are not the ones `value` comes from
    pairs = [(new_event(), new_event()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in pairs:
        lay.step([None, None, None, None, a, b, None, None, None])
    torch.cuda.synchronize()
    ev_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    w13_ms = float(np.mean([elapsed_ms(a, b) for a, b in pairs]))
    own_events = [e for p in pairs for e in p]

    active, layer_bytes, flops, w13_bytes, w13_flops = algorithmic(spec, counts)
    peak = MFMA_PEAK_TFLOPS[mode]
    (type13, peak13), (_, peak2) = issued_mfma(mode, lay.big)
    issued_roof_ms = (w13_flops / (peak13 * 1e12) + (flops - w13_flops) / (peak2 * 1e12)) * 1e3
    w13_gbs = w13_bytes / (w13_ms * 1e-3) / 1e9
    w13_tflops = w13_flops / (w13_ms * 1e-3) / 1e12
    # the dominant kernel's binding roof: HBM below the ridge of the layer's
    # MFMA type (peak flops / 8 TB/s), MFMA above it
    mfma_bound = w13_flops / w13_bytes > peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    roofline = {"bound": "mfma" if mfma_bound else "hbm", "kernel": lay.kernel,
                "achieved": w13_tflops if mfma_bound else w13_gbs,
                "peak": peak if mfma_bound else HBM_PEAK_GBS,
                "unit": "TFLOP/s" if mfma_bound else "GB/s",
                "frac": w13_tflops / peak if mfma_bound else w13_gbs / HBM_PEAK_GBS,
                "traffic": traffic_for(spec.name, lay.kernel, kernel_sources(lay.big)),
                "bytes_per_launch": w13_bytes, "flops_per_launch": w13_flops, "avg_ms": w13_ms,
                "hbm_gbs": w13_gbs, "mfma_tflops": w13_tflops, "mfma_peak_tflops": peak,
                "mfma_issued": type13,
                "mfma_frac_of_issued_type_peak": w13_tflops / peak13}
    rec = {
        "workload": "%s: T=%d H=%d E=%d k=%d I=%d" % (spec.name, spec.T, spec.H, spec.E, spec.k,
                                                     spec.I),
        "dtype": DTYPE_NAME[mode],
        "ms_per_step": ms,
        "ms_per_step_kernel_timed": ev_ms,
        "tokens_per_s": spec.T / (ms * 1e-3),
        "active_experts": active,
        "layer_hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
        "layer_hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "layer_tflops": flops / (ms * 1e-3) / 1e12,
        "layer_mfma_frac": flops / (ms * 1e-3) / 1e12 / peak,
        "layer_mfma_frac_issued": issued_roof_ms / ms,
        "mfma_types": {"gate_up": type13, "down": issued_mfma(mode, lay.big)[1][0]},
        "layer_alg_bytes": layer_bytes,
        "layer_alg_flops": flops,
        "roofline": roofline,
    }
    # the layer from the router weights (a separate figure): the same steps
    # from x and the router weights (moe_fused_forward_router: for few-token
    # bf16/FP8 batches the front kernel computes the logits itself), and the
    # router GEMM alone (moe_router_logits)
    lg = torch.empty((spec.T, spec.E), dtype=torch.float32, device="cuda")

    def router_step():
        moe.moe_fused_forward_router(lay.x, lay.wg, lay.w13, lay.s13, lay.w2, lay.s2, spec.k,
                                     out=lay.out, ws=lay.ws, topk_ids=lay.ids)

    for _ in range(args.warmup):
        router_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        router_step()
    torch.cuda.synchronize()
    router_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ra, rb = new_event(), new_event()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    H_.hipEventRecord(ctypes.c_void_p(ra), stream)
    for _ in range(args.steps):
        moe.moe_router_logits(lay.x, lay.wg, k=spec.k, ws=lay.ws, logits=lg)
    H_.hipEventRecord(ctypes.c_void_p(rb), stream)
    torch.cuda.synchronize()
    router_ms = elapsed_ms(ra, rb) / args.steps
    own_events += [ra, rb]
    rec["router"] = {"ms_per_step": router_step_ms,
                     "tokens_per_s": spec.T / (router_step_ms * 1e-3),
                     "router_gemm_ms": router_ms}
    if full:
        # the same step replayed from a captured HIP graph (a separate,
        # labelled figure: launches without per-launch CPU work; `value`
        # stays the eagerly launched rate)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            lay.step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        del graph

        # single calls after an L2 / MALL flush (outside the timed region):
        # the flush only reads, so the timed call inherits no dirty lines
        flush_buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        # 100 calls for the few-token (decode) layers, 20 for the tiled ones
        fpairs = [(new_event(), new_event()) for _ in range(20 if lay.big else 100)]
        for a, b in fpairs:
            flush_buf.sum()
            lay.step([a, None, None, None, None, None, None, None, b])
        torch.cuda.synchronize()
        fms = np.array([elapsed_ms(a, b) for a, b in fpairs])
        del flush_buf

        # per-stage breakdown (outside the timed region; every boundary)
        evs = [new_event() for _ in range(moe.NUM_STAGE_EVENTS)]
        reps = min(args.steps, 20)
        stage_ms = np.zeros(moe.NUM_STAGE_EVENTS - 1)
        for _ in range(reps):
            lay.step(evs)
            H_.hipEventSynchronize(ctypes.c_void_p(evs[-1]))
            stage_ms += [elapsed_ms(evs[i], evs[i + 1]) for i in range(moe.NUM_STAGE_EVENTS - 1)]
        stage_ms /= reps
        own_events += evs + [e for p in fpairs for e in p]
        rec.update({
            "graph_replay": {"ms_per_step": graph_ms, "tokens_per_s": spec.T / (graph_ms * 1e-3),
                             "layer_hbm_frac": layer_bytes / (graph_ms * 1e-3) / 1e9 /
                             HBM_PEAK_GBS},
            "flushed": {"calls": len(fms), "ms_median": float(np.median(fms)),
                        "ms_p10": float(np.percentile(fms, 10)),
                        "ms_p90": float(np.percentile(fms, 90)),
                        "layer_hbm_frac_median": layer_bytes / (np.median(fms) * 1e-3) / 1e9 /
                        HBM_PEAK_GBS},
            "stage_ms": {n: round(float(v), 5) for n, v in zip(
                ["gating", "align_sort", "tiles", "x_quant", "w13_swiglu", "h_quant", "w2",
                 "combine"], stage_ms)},
        })
    for e in own_events:
        H_.hipEventDestroy(ctypes.c_void_p(e))
    rec["_layer"] = lay
    return rec


def measure_rope(name, args, H_):
    """Time K launches of the inverse rotary embedding + per-head FP8
    quantisation step (moe_inv_rope_fp8_quant) on a seeded batch; the
    kernel's duration comes from an event pair around the K launches on the
    launch stream.  Algorithmic bytes: x read once (2 B per value), codes
    written (1 B per value), one fp32 scale per (token, head), the positions,
    and the table rows of the batch's distinct positions."""
    import numpy as np
    import torch

    import moe_layer_gating_amd as moe
    import moe_workloads as wl

    spec = wl.ROPE_WORKLOADS[name]
    log("generating", name)
    R = wl.make_rope(spec)
    x = torch.from_numpy(R["x"].view(np.int16)).view(torch.bfloat16).cuda()
    pos = torch.from_numpy(R["positions"]).cuda()
    cs = torch.from_numpy(R["cos_sin"]).cuda()
    T, nh, hd, rot = spec.T, spec.n_heads, spec.head_dim, spec.rot_dim
    codes = torch.empty((T, nh, hd), dtype=torch.uint8, device="cuda")
    scales = torch.empty((T, nh), dtype=torch.float32, device="cuda")

    def launch():
        moe.moe_inv_rope_fp8_quant(x, pos, cs, interleaved=spec.interleaved, codes=codes,
                                   scales=scales)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    e = [ctypes.c_void_p(), ctypes.c_void_p()]
    for ev in e:
        assert H_.hipEventCreate(ctypes.byref(ev)) == 0
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    reps = max(args.steps, 50)
    t0 = time.perf_counter()
    H_.hipEventRecord(e[0], stream)
    for _ in range(reps):
        launch()
    H_.hipEventRecord(e[1], stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / reps
    f = ctypes.c_float()
    assert H_.hipEventElapsedTime(ctypes.byref(f), e[0], e[1]) == 0
    for ev in e:
        H_.hipEventDestroy(ev)
    ms = f.value / reps
    n_pos = int(np.unique(R["positions"]).size)
    nbytes = T * nh * hd * 3 + T * nh * 4 + T * 4 + n_pos * rot * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "%s: T=%d heads=%d head_dim=%d rot_dim=%d max_pos=%d" % (
                name, T, nh, hd, rot, spec.max_pos),
            "dtype": "bf16 in, fp8e4m3 out", "ms_per_launch": ms, "wall_ms_per_launch": wall,
            "tokens_per_s": T / (ms * 1e-3), "alg_bytes": nbytes,
            "roofline": {"bound": "hbm", "kernel": "inv_rope_fp8_kernel", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": traffic_for(name, "inv_rope_fp8_kernel", ROPE_SOURCES)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_fp8")
    ap.add_argument("--sub", default="decode_bf16,rope_prefill",
                    help="comma-separated layers (or rope_prefill / rope_decode, the inverse "
                         "rotary embedding + FP8 step) measured as sub-records, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (the reference "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this layer is built and measured on a single "
              "MI355X (no sharding or collectives); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n,
                          "launches": 5}), flush=True)
        return

    H_ = hip()
    main_rec = measure(args.workload, args, H_, full=True)
    lay = main_rec.pop("_layer")
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(lay.L)
    spec = lay.spec
    del lay
    gc.collect()
    torch.cuda.empty_cache()

    subs = {}
    for name in [n for n in args.sub.split(",") if n and n != "none" and n != args.workload]:
        if name.startswith("rope_"):
            subs[name] = measure_rope(name, args, H_)
            continue
        r = measure(name, args, H_, full=False)
        del r["_layer"]
        gc.collect()
        torch.cuda.empty_cache()
        subs[name] = r

    rec = {
        "metric": METRIC,
        "value": main_rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_NAME[spec.mode],
        # the MFMA arithmetic each GEMM issues
        "mfma_types": main_rec["mfma_types"],
        "data": "synthetic (seeded; moe_workloads recipe)",
        "config": {"workload": main_rec["workload"], "T": spec.T, "H": spec.H, "E": spec.E,
                   "k": spec.k, "I": spec.I, "active_experts": main_rec["active_experts"]},
    }
    for key in ("layer_hbm_gbs", "layer_hbm_frac", "layer_tflops", "layer_mfma_frac",
                "layer_mfma_frac_issued", "layer_alg_bytes", "layer_alg_flops", "graph_replay",
                "router", "flushed", "stage_ms", "roofline"):
        rec[key] = main_rec[key]
    rec["cpu_baseline"] = cpu
    rec["sub_records"] = subs
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
