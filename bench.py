"""Benchmark of the FP8 (e4m3) weight-only linear layer on one MI355X.

One step = one pass of the per-call hot path for M = 1..32 over the weight
shapes the metric names:
  * the decode GEMV workload, M = 1: three fp8w_linear calls with bf16
    activations and a zero bf16 bias on the weights [4096, 4096],
    [14336, 4096] and [4096, 14336] (N(0, 0.02^2) fp32, quantized once per
    output channel); these run the M = 1 GEMV (gemv_kernel);
  * the skinny sweep, M = 2, 4, 8, 16, 22, 32: six fp8w_linear calls with
    fp16 activations and an N(0, 0.01^2) fp16 bias on [14336, 4096]
    (0.02 * Student-t(3) weights); these run the matrix-core skinny GEMM
    (pipe_kernel).
Every weight was quantized once at build time (not timed here). Inputs are
resident in HBM when the timed region starts, and every call reads a different
copy of its weight codes and scales (each layer's copies rotate through
>= 1 GiB), so the 256 MB Infinity Cache cannot serve repeats: the kernels
stream from HBM.

The timed region launches the K steps eagerly through the C ABI (ctypes) on
torch's current stream: first the K steps' M = 1 calls, then their M >= 2
calls, with one HIP event at the start, one between the two phases and one at
the end (synchronizes on both sides). The work is the K steps' work; the
phase order only lets each kernel family's mean launch time be read from the
events without a marker per step. If K steps take less than --min-ms, the
region is timed again with enough steps to last that long; "steps" is the
number of steps actually timed ("steps_requested" is K).

value = algorithmic bytes of the timed steps / the timed region's duration, in
GB/s. Algorithmic bytes per call = N*K (codes) + 4N (scales) + 2N (bias) +
2MK (x) + 2MN (y).

roofline: for the kernel family that takes most of the step's time, achieved =
its algorithmic bytes per launch / its mean launch duration (its phase of the
timed region divided by its launches), against 8 TB/s; "kernels" gives the
same for both families. traffic = HBM bytes per launch from the committed
rocprofv3 --pmc summary (profiles/step_traffic.json), reported only while the
family's sources and the library's compile flags hash to the value recorded
there.

Every timed region is preceded by --spin-ms of the same work: the GPU raises
its clocks only under sustained load, and the first ~10 ms run up to 15 %
slower than the steady state measured here.

stdout: ONE compact JSON line (the headline: the metric, the timed region, the
roofline, per-call microseconds from back-to-back bursts of each call, the
streaming-read reference, and the CPU oracle baseline). Progress goes to
stderr, and the full record (per-call percentiles, warm numbers, host latency,
the oracle timed on every workload and, with --extra, the other workloads) is
written to --full-json (default results/bench_full.json).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--min-ms MS] [--spin-ms MS]
                       [--extra] [--only tiny|skinny|block|large|batch|grouped|w8a8 ...] [--reps R]
Profiler helpers: --only-timed (the timed region alone), --shape N K M [--act fp16] (one call
shape alone), --trace-summary CSV [--last N],
--mfma-summary CSV N K, --pmc-summary FETCH_CSV WRITE_CSV, --counter-summary KERNEL CSV [CSV ...].
"""
import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import fp8_weight_only_amd as fw  # noqa: E402
import workloads  # noqa: E402

METRIC = "fp8-weight linear achieved HBM GB/s (% of peak) + µs/call, M=1..32, K,N=4096..8192"
DTYPE = "bf16/fp16 x e4m3 -> f32 acc"
PEAK_HBM_GBPS = 8000.0
ROTATE_BYTES = 1 << 30
SPIN_MS = 200.0  # sustained load before every timed region (clock ramp-up); --spin-ms
MIN_TIMED_MS = 50.0  # shortest timed region; --min-ms
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_traffic.json")
FULL_RECORD = os.path.join(ROOT, "results", "bench_full.json")

# the kernel families of the step and the sources that define each (kernel code
# and tile choice): a change to any of them, or to the compile flags, voids that
# family's recorded traffic
FAMILIES = {"gemv_kernel": ("common.hpp", "gemv.hip"),
            "pipe_kernel": ("common.hpp", "ring.hpp", "skinny.hip")}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(m, n, k, bias=True):
    return n * k + 4 * n + (2 * n if bias else 0) + 2 * m * k + 2 * m * n


def kernel_source_hash(family):
    from fp8_weight_only_amd import _build
    flags = [f for f in _build.CFLAGS if not f.startswith("--offload-arch") and not os.path.isabs(f) and f != "-I"]
    h = hashlib.sha256(" ".join(flags).encode())  # the compile flags shape the code too (paths left out)
    d = os.path.join(ROOT, "fp8_weight_only_amd", "csrc")
    for f in FAMILIES[family]:
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class Layer:
    """One quantized layer on the GPU with `copies` rotated copies of (q, scale)."""

    def __init__(self, lw, copies, dev):
        w = torch.from_numpy(lw.w).to(dev)
        fw.quantize(w)  # first call also loads the code object
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        q, s = fw.quantize(w)  # kernel + scale read-back + stream sync
        self.quantize_ms = (time.perf_counter() - t0) * 1e3
        self.n, self.k = lw.w.shape
        self.name = lw.name
        del w
        self.qs = [(q, s)] + [(q.clone(), s.clone()) for _ in range(copies - 1)]
        self.bias = None if lw.bias is None else lw.bias.to(dev)


class GroupedLayer:
    """A layer quantized with group scales along k, `copies` rotated copies."""

    def __init__(self, lw, group, copies, dev):
        w = torch.from_numpy(lw.w).to(dev)
        fw.quantize_grouped(w, group)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        q, s = fw.quantize_grouped(w, group)
        self.quantize_ms = (time.perf_counter() - t0) * 1e3
        self.n, self.k = lw.w.shape
        self.group = group
        self.name = f"{lw.name}_g{group}"
        del w
        self.qs = [(q, s)] + [(q.clone(), s.clone()) for _ in range(copies - 1)]
        self.bias = None if lw.bias is None else lw.bias.to(dev)


def grouped_bytes(m, n, k, g, bias):
    return n * k + 4 * n * (k // g) + (2 * n if bias else 0) + 2 * m * k + 2 * m * n


class GroupedCall:
    """One grouped call per weight copy; a batch plan that splits k gets the
    workspace it asks for (fp8w_linear_grouped_with_workspace)."""

    def __init__(self, layer, x, dev):
        self.layer, self.x = layer, x
        self.m = x.shape[0]
        self.y = torch.empty((self.m, layer.n), dtype=x.dtype, device=dev)
        act = fw.BF16 if x.dtype == torch.bfloat16 else fw.FP16
        self.act = act
        need = fw.fp8w_linear_grouped_workspace_bytes(self.m, layer.n, layer.k, layer.group, act, x.data_ptr(),
                                                      layer.qs[0][0].data_ptr())
        self.ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        self.args = [(x.data_ptr(), act, self.m, layer.k, q.data_ptr(), s.data_ptr(), layer.group,
                      0 if layer.bias is None else layer.bias.data_ptr(), layer.n, self.y.data_ptr(),
                      self.ws.data_ptr() if need else 0, need, fw.PATH_AUTO)
                     for q, s in layer.qs]
        self.bytes = grouped_bytes(self.m, layer.n, layer.k, layer.group, layer.bias is not None)
        self.kernel = fw.fp8w_linear_grouped_kernel(fw.PATH_AUTO, self.m, layer.n, layer.k, layer.group, act,
                                                    x.data_ptr(), layer.qs[0][0].data_ptr())

    def launch(self, copy, stream):
        r = fw.load().fp8w_linear_grouped_with_workspace(*self.args[copy % len(self.args)], stream)
        if r != 0:
            raise fw.Fp8wError(r, "fp8w_linear_grouped_with_workspace")


def grouped_report(call, st):
    us = st["mean"]
    gbps = call.bytes / (us * 1e-6) / 1e9
    useful = 2.0 * call.m * call.layer.n * call.layer.k
    r = {"layer": call.layer.name, "group": call.layer.group, "m": call.m, "n": call.layer.n, "k": call.layer.k,
         "kernel": call.kernel, "us_per_call": round(us, 3), "us_p10": round(st["p10"], 3),
         "us_p90": round(st["p90"], 3), "alg_bytes": call.bytes, "gbps": round(gbps, 1),
         "pct_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
         "tflops": round(useful / (us * 1e-6) / 1e12, 3)}
    issued, mpad = mfma_issued_flops(call.kernel, call.m, call.layer.n, call.layer.k)
    if issued:
        r["mfma"] = {"padded_m": mpad, "issued_pct_of_peak": round(100.0 * issued / (us * 1e-6) / 1e12 /
                                                                   MFMA_PEAK_TFLOPS, 3),
                     "useful_pct_of_peak": round(100.0 * useful / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 3)}
    return r


class Call:
    """Argument tuples of one fp8w_linear call for every weight copy (path:
    fp8w_linear_with_path's forced path instead of the dispatch's)."""

    def __init__(self, layer, x, dev, ws=None, path=None):
        self.layer, self.x = layer, x
        self.m = x.shape[0]
        self.req_path = fw.PATH_AUTO if path is None else path
        self.y = torch.empty((self.m, layer.n), dtype=x.dtype, device=dev)
        act = fw.BF16 if x.dtype == torch.bfloat16 else fw.FP16
        if ws is None:  # the workspace the library asks for (fallback, or a k split), allocated once
            wsb = fw.fp8w_linear_with_path_workspace_bytes(self.req_path, self.m, layer.n, layer.k, act,
                                                           x.data_ptr(), layer.qs[0][0].data_ptr())
            ws = torch.empty((wsb,), dtype=torch.uint8, device=dev) if wsb else None
        self.ws = ws
        self.path = ["gemv", "skinny", "fallback", "batch"][
            fw.linear_path(x, layer.qs[0][0]) if path is None else path]
        self.args = [(x.data_ptr(), act, self.m, layer.k, q.data_ptr(), s.data_ptr(),
                      0 if layer.bias is None else layer.bias.data_ptr(), layer.n, self.y.data_ptr(),
                      0 if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel())
                     for q, s in layer.qs]
        self.bytes = alg_bytes(self.m, layer.n, layer.k, layer.bias is not None)

    def launch(self, copy, stream):
        if self.req_path == fw.PATH_AUTO:
            r = fw.load().fp8w_linear(*self.args[copy % len(self.args)], stream)
        else:
            r = fw.load().fp8w_linear_with_path(*self.args[copy % len(self.args)], self.req_path, stream)
        if r != 0:
            raise fw.Fp8wError(r, "fp8w_linear")


FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense e4m3 matrix-core peak


class W8Call:
    """One W8A8 call over rotated weight copies: the whole layer
    (fp8w_linear_w8a8: per-token quantize of x, then the fp8 GEMM), the GEMM
    alone on x quantized once (fp8w_gemm_w8a8), or the activation quantizer
    alone (fp8w_quantize_activations)."""

    def __init__(self, layer, x, dev, mode):
        self.layer, self.x, self.mode = layer, x, mode
        self.m = x.shape[0]
        m, n, k = self.m, layer.n, layer.k
        self.y = torch.empty((m, n), dtype=x.dtype, device=dev)
        self.ws = torch.empty((fw.fp8w_linear_w8a8_workspace_bytes(m, k),), dtype=torch.uint8, device=dev)
        self.qx, self.sx = fw.quantize_activations(x)
        act = fw.BF16 if x.dtype == torch.bfloat16 else fw.FP16
        lib = fw.load()
        if mode == "layer":
            self.fn = lib.fp8w_linear_w8a8
            self.args = [(x.data_ptr(), act, m, k, q.data_ptr(), s.data_ptr(), 0, n, self.y.data_ptr(),
                          self.ws.data_ptr(), self.ws.numel()) for q, s in layer.qs]
        elif mode == "gemm":
            self.fn = lib.fp8w_gemm_w8a8
            self.args = [(self.qx.data_ptr(), self.sx.data_ptr(), m, k, q.data_ptr(), s.data_ptr(), 0, n,
                          self.y.data_ptr(), act) for q, s in layer.qs]
        else:
            self.fn = lib.fp8w_quantize_activations
            self.args = [(x.data_ptr(), act, m, k, self.qx.data_ptr(), self.sx.data_ptr())]
        self.kernel = fw.fp8w_linear_w8a8_kernel(m, n, k)

    def launch(self, copy, stream):
        r = self.fn(*self.args[copy % len(self.args)], stream)
        if r != 0:
            raise fw.Fp8wError(r, self.fn.__name__)


def w8a8_report(call, st):
    us = st["mean"]
    m, n, k = call.m, call.layer.n, call.layer.k
    r = {"layer": call.layer.name, "mode": call.mode, "m": m, "n": n, "k": k, "us_per_call": round(us, 3),
         "us_p10": round(st["p10"], 3), "us_p90": round(st["p90"], 3)}
    if call.mode == "quantize_x":
        moved = 2 * m * k + m * k + 4 * m
        r.update(gbps=round(moved / (us * 1e-6) / 1e9, 1),
                 pct_peak=round(100.0 * moved / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2))
    else:
        tf = 2.0 * m * n * k / (us * 1e-6) / 1e12
        r.update(kernel=call.kernel, tflops=round(tf, 1), pct_fp8_peak=round(100.0 * tf / FP8_MFMA_PEAK_TFLOPS, 2))
    return r


def spin_up(launch, ms):
    """Run `launch(i)` back to back for at least `ms` milliseconds of wall time.
    The GPU's power management raises its clocks only under sustained load:
    measured here, the first ~10 ms of a burst run up to 15 % slower than the
    steady state, so every timed region is preceded by this much of its own work."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(32):
            launch(i)
            i += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return i


def burst(call, reps, warmup, stream, warm=False, spin_ms=None, groups=10):
    """Microseconds per launch over `reps` back-to-back launches of one call
    (rotating weight copies unless warm), between events on the launch stream.
    The launches are split into `groups` equal groups, each between two events:
    "mean" is the whole burst's average, "p10" / "median" / "p90" are taken over
    the groups' averages."""
    spin_up(lambda i: call.launch(0 if warm else i, stream), SPIN_MS if spin_ms is None else spin_ms)
    for i in range(warmup):
        call.launch(0 if warm else i, stream)
    torch.cuda.synchronize()
    groups = max(1, min(groups, reps))
    per = reps // groups
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    ev[0].record()
    i = 0
    for g in range(groups):
        for _ in range(per):
            call.launch(0 if warm else i, stream)
            i += 1
        ev[g + 1].record()
    torch.cuda.synchronize()
    gus = np.array([ev[g].elapsed_time(ev[g + 1]) * 1e3 / per for g in range(groups)])
    return {"mean": ev[0].elapsed_time(ev[groups]) * 1e3 / (per * groups),
            "p10": float(np.percentile(gus, 10)), "median": float(np.median(gus)),
            "p90": float(np.percentile(gus, 90))}


def burst_us(call, reps, warmup, stream, warm=False, spin_ms=None):
    return burst(call, reps, warmup, stream, warm, spin_ms)["mean"]


def host_latency(call, stream, reps=200):
    """Host wall time of one warm call (same weight copy every time): the ctypes
    call into fp8w_linear alone (enqueue), and the call followed by a stream
    synchronize (the latency a caller that waits for the result sees), medians
    over `reps` calls."""
    call.launch(0, stream)
    torch.cuda.synchronize()
    enq, full = [], []
    for _ in range(reps):
        t0 = time.perf_counter()
        call.launch(0, stream)
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        enq.append(t1 - t0)
        full.append(t2 - t0)
    return {"enqueue_us": round(float(np.median(enq)) * 1e6, 2),
            "call_and_sync_us": round(float(np.median(full)) * 1e6, 2), "calls": reps}


MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 matrix-core peak of MI355X


def mfma_issued_flops(kernel, m, n, k):
    """Matrix-core FLOPs a skinny launch issues, from its tile parameters (the
    kernel name fp8w_linear_kernel reports): every v_mfma_f32_16x16x32 is
    2*16*16*32 FLOPs whether its token columns are real or padding.
    pipe_kernel: 16*CT-channel blocks, tokens padded to 16*MT (MT = 2 above 16
    rows); seg_kernel: MP = 16/SEG channels x MP tokens per segment, SEG
    segments per instruction of which one is kept, so tokens count as
    MP*MT*SEG. None for other kernels."""
    import re
    mm = re.match(r"pipe(?:_grouped)?_kernel<XR=(\d+),CT=(\d+),KP=\d+,NS=\d+(?:,CB=(\d+))?>", kernel or "")
    if mm:
        xr, ct = int(mm.group(1)), int(mm.group(2))
        cb = int(mm.group(3) or 16)
        mt = 2 if xr > 16 else 1
        chans = 16 * ct * math.ceil(n / (16 * ct))
        cols = k
        if cb != 16:  # the ring's columns (an even number of stages), then 32-column MFMA blocks for the rest
            room = k - 8 if cb == 8 and k % 16 == 8 else k
            kr = room - room % 256
            kr -= 256 if (kr // 256) % 2 else 0
            cols = kr + 32 * math.ceil((k - kr) / 32)
            if cb == 8:  # workgroups of one row parity, a pair per 32 * CT channels; an odd one past n exits
                pairs = math.ceil(n / (32 * ct))
                chans = 16 * ct * (2 * pairs - (1 if 32 * ct * (pairs - 1) + 1 >= n else 0))
        return 2.0 * cols * chans * 16 * mt, 16 * mt
    mm = re.match(r"seg_kernel<SEG=(\d+),T=(\d+),W=\d+,U=\d+,MT=(\d+)>", kernel or "")
    if mm:
        seg, t, mt = int(mm.group(1)), int(mm.group(2)), int(mm.group(3))
        mp = 16 // seg
        chans = mp * t * math.ceil(n / (mp * t))
        return 2.0 * k * chans * mp * mt * seg, mp * mt * seg
    return None, None


def call_report(call, us):
    """Per-call line: `us` is a burst() result (or a plain mean in microseconds)."""
    st = us if isinstance(us, dict) else None
    us = st["mean"] if st else us
    gbps = call.bytes / (us * 1e-6) / 1e9
    act = fw.BF16 if call.x.dtype == torch.bfloat16 else fw.FP16
    kernel = fw.fp8w_linear_kernel(getattr(call, "req_path", fw.PATH_AUTO), call.m, call.layer.n, call.layer.k,
                                   act, call.x.data_ptr(), call.layer.qs[0][0].data_ptr())
    if call.path in ("skinny", "batch") and call.ws is None and "splitk" in kernel:
        kernel = "single pass (no workspace)"
    useful = 2.0 * call.m * call.layer.n * call.layer.k
    r = {"layer": call.layer.name, "m": call.m, "n": call.layer.n, "k": call.layer.k, "path": call.path,
         "kernel": kernel,
         "us_per_call": round(us, 3), "alg_bytes": call.bytes, "gbps": round(gbps, 1),
         "pct_peak": round(100.0 * gbps / PEAK_HBM_GBPS, 2),
         "tflops": round(useful / (us * 1e-6) / 1e12, 3)}
    if st:
        r["us_p10"], r["us_median"], r["us_p90"] = (round(st[q], 3) for q in ("p10", "median", "p90"))
    if call.path == "skinny":
        issued, mpad = mfma_issued_flops(kernel, call.m, call.layer.n, call.layer.k)
        if issued:
            r["mfma"] = {"padded_m": mpad, "issued_tflops": round(issued / (us * 1e-6) / 1e12, 2),
                         "useful_pct_of_peak": round(100.0 * useful / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 3),
                         "issued_pct_of_peak": round(100.0 * issued / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 3)}
    return r


def capture_pass(calls, copies, stream_obj):
    """One HIP graph holding `copies` steps, step c on weight copy c (every call
    once per step): one replay is one pass over the rotated copies."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream_obj):
        st = torch.cuda.current_stream().cuda_stream
        for c in range(copies):
            for call in calls:
                call.launch(c, st)
    return g


def timed_steps(calls, steps, warmup, copies, use_graph, dev):
    """Duration (ms) of exactly `steps` steps, events around them and synchronizes
    on both sides. With use_graph the steps are replays of one pass graph, so
    `steps` must be a multiple of `copies`."""
    stream = torch.cuda.current_stream(dev)
    graph = None
    if use_graph:
        if steps % copies:
            raise ValueError("graph steps must be a whole number of passes over the weight copies")
        graph = capture_pass(calls, copies, torch.cuda.Stream(device=dev))
    torch.cuda.synchronize()

    def step(i):
        for call in calls:
            call.launch(i, stream.cuda_stream)

    def unit(i):  # one eager step, or one replayed pass of `copies` steps
        if graph is not None:
            graph.replay()
        else:
            step(i)

    per_unit = copies if graph is not None else 1
    spin_up(unit, SPIN_MS)
    for i in range(-(-warmup // per_unit)):
        unit(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps // per_unit):
        unit(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


class Step:
    """The timed workload: the three M = 1 decode calls and the six skinny-sweep
    calls (M = 2..32) of one step, each layer with enough weight copies that a
    copy is read again only after >= 1 GiB of other weights."""

    def __init__(self, dev):
        self.dec_lws = [workloads.decode_layer(i) for i in range(len(workloads.DECODE_SHAPES))]
        dec_bytes = sum(lw.w.shape[0] * lw.w.shape[1] for lw in self.dec_lws)
        self.dec_copies = max(1, math.ceil(ROTATE_BYTES / dec_bytes))
        self.dec_layers = [Layer(lw, self.dec_copies, dev) for lw in self.dec_lws]
        self.dec_xs = [workloads.decode_x(i) for i in range(len(self.dec_lws))]
        self.dec_calls = [Call(L, x.to(dev), dev) for L, x in zip(self.dec_layers, self.dec_xs)]
        self.sk_lw = workloads.skinny_layer()
        n, k = self.sk_lw.w.shape
        self.sk_copies = max(1, math.ceil(ROTATE_BYTES / (n * k)))
        self.sk_layer = Layer(self.sk_lw, self.sk_copies, dev)
        self.sk_xs = [workloads.skinny_x(m) for m in workloads.SKINNY_MS]
        self.sk_calls = [Call(self.sk_layer, x.to(dev), dev) for x in self.sk_xs]
        self.calls = self.dec_calls + self.sk_calls
        self.dec_step_bytes = sum(c.bytes for c in self.dec_calls)
        self.sk_step_bytes = sum(c.bytes for c in self.sk_calls)
        self.step_bytes = self.dec_step_bytes + self.sk_step_bytes

    def gemv_phase(self, i0, count, stream):
        for i in range(i0, i0 + count):
            for c in self.dec_calls:
                c.launch(i, stream)

    def skinny_phase(self, i0, count, stream):
        per = len(self.sk_calls)
        for i in range(i0, i0 + count):
            for j, c in enumerate(self.sk_calls):
                c.launch(i * per + j, stream)


def timed_region(step, steps, warmup, dev, spin=True):
    """(ms of the M = 1 phase, ms of the M >= 2 phase) of exactly `steps` steps:
    events on the launch stream at the start, between the phases and at the end,
    synchronizes on both sides."""
    stream = torch.cuda.current_stream(dev).cuda_stream
    if spin:
        spin_up(lambda i: (step.gemv_phase(i, 1, stream), step.skinny_phase(i, 1, stream)), SPIN_MS)
    step.gemv_phase(0, warmup, stream)
    step.skinny_phase(0, warmup, stream)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    step.gemv_phase(0, steps, stream)
    ev[1].record()
    step.skinny_phase(0, steps, stream)
    ev[2].record()
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])


def read_ceiling(dev, sizes, reps=100):
    """The library's plain streaming-read kernel over the same byte counts,
    rotating through 1 GiB: the reference the GEMV's bandwidth is read against."""
    big = torch.empty(ROTATE_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    out = []
    for nbytes in sizes:
        copies = max(1, big.numel() // nbytes)

        def go(i):
            st = fw.fp8w_stream_read_probe(big.data_ptr() + (i % copies) * nbytes, nbytes, sink.data_ptr(), stream)
            if st != 0:
                raise fw.Fp8wError(st, "fp8w_stream_read_probe")
        spin_up(go, SPIN_MS)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(reps):
            go(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out.append({"bytes": nbytes, "us": round(us, 3), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                    "pct_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2)})
    del big
    torch.cuda.empty_cache()
    return out


def cpu_info():
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                model = line.split(":", 1)[1].strip()
    except Exception:  # noqa: BLE001
        pass
    return os.cpu_count(), model


def cpu_baseline(step, budget_s):
    """The oracle (fp64 C, OpenMP over output channels) on the host cores, on the
    same nine calls of one step, repeated until ~budget_s of CPU work; then the
    three M = 1 calls on one core. The oracle's results of this leg are also
    compared with the GPU's: codes and scales bit for bit, and the GPU outputs
    of the same calls against the output gate."""
    import oracle
    quant = {}
    for lw in step.dec_lws + [step.sk_lw]:
        q, s, st = oracle.quantize_rows(lw.w)
        quant[lw.name] = (q, s, oracle.row_amax(lw.w), st)
    prepared = []
    for c, lw, x in zip(step.calls, step.dec_lws + [step.sk_lw] * len(step.sk_calls), step.dec_xs + step.sk_xs):
        q, s, amax, _ = quant[lw.name]
        prepared.append((c, lw, x.double().numpy(), q, s, None if lw.bias is None else lw.bias.double().numpy(),
                         amax))

    def run(items, budget):
        reps, byts, outs = 0, 0, []
        t0 = time.perf_counter()
        while True:
            outs = []
            for (_, _, x64, q, s, b, _) in items:
                outs.append(oracle.linear_f64(x64, q, s, b))
                byts += alg_bytes(x64.shape[0], q.shape[0], q.shape[1], b is not None)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, byts, el, outs

    threads = oracle.num_threads()
    reps, byts, el, outs = run(prepared, budget_s)
    oracle.set_num_threads(1)
    try:
        reps1, byts1, el1, _ = run(prepared[:len(step.dec_calls)], min(budget_s, 3.0))
    finally:
        oracle.set_num_threads(threads)

    # parity of this run's GPU results against the oracle's
    ok = True
    for L in step.dec_layers + [step.sk_layer]:
        q, s, _, st = quant[L.name]
        ok &= st == 0
        ok &= bool(np.array_equal(L.qs[0][0].cpu().numpy(), q))
        ok &= bool(np.array_equal(L.qs[0][1].cpu().numpy().view(np.uint32), s.view(np.uint32)))
    for (c, _, x64, _, _, _, amax), y_ref in zip(prepared, outs):
        c.y.fill_(float("nan"))
        c.launch(0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        yv = c.y.double().cpu().numpy()
        tol = 1e-2 * np.abs(y_ref) + 1e-3 * np.linalg.norm(x64, axis=1)[:, None] * amax[None, :]
        ok &= bool(np.all(np.isfinite(yv)) and np.all(np.abs(yv - y_ref) <= tol))

    nproc, model = cpu_info()
    return {"value": round(byts / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} passes over one step's 9 calls (3 decode GEMVs at M=1, the skinny sweep at "
                      f"M=2..32) through the fp64 oracle, {el:.1f} s",
            "one_core": {"value": round(byts1 / el1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                         "sample": f"{reps1} passes over the 3 decode calls, {el1:.1f} s"},
            "gpu_parity_vs_this_oracle_run": ok, "host_cpus": nproc, "host_model": model}


def oracle_per_config():
    """The oracle's quantizer and fp64 linear timed on every workload (part of the
    cpu_baseline leg): median wall time of `reps` runs on all host threads, and
    for the smaller workloads again on one thread. GB/s use the same algorithmic
    bytes as the GPU lines (the quantizer: 4 B read + 1 B written per weight)."""
    import oracle
    threads = oracle.num_threads()

    def med(fn, reps):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    def one(name, lw, xs, reps, one_core):
        n, k = lw.w.shape
        q, s, _ = oracle.quantize_rows(lw.w)
        b = None if lw.bias is None else lw.bias.double().numpy()
        r = {"workload": name, "n": n, "k": k, "runs": reps}
        tq = med(lambda: oracle.quantize_rows(lw.w), reps)
        r["quantize_us"] = round(tq * 1e6, 1)
        r["quantize_gbps"] = round(5.0 * n * k / tq / 1e9, 3)
        r["linear"] = []
        for x in xs:
            x64 = x.double().numpy()
            m = x64.shape[0]
            byts = alg_bytes(m, n, k, b is not None)
            t = med(lambda: oracle.linear_f64(x64, q, s, b), reps)
            e = {"m": m, "us": round(t * 1e6, 1), "gbps": round(byts / t / 1e9, 3)}
            if one_core:
                oracle.set_num_threads(1)
                try:
                    t1 = med(lambda: oracle.linear_f64(x64, q, s, b), 1)
                finally:
                    oracle.set_num_threads(threads)
                e["one_core_us"] = round(t1 * 1e6, 1)
                e["one_core_gbps"] = round(byts / t1 / 1e9, 3)
            r["linear"].append(e)
        return r

    out = []
    t0 = time.perf_counter()
    case = workloads.tiny_gemv()
    out.append(one("tiny", case.layer, [case.x], 10, True))
    for i in range(3):
        out.append(one("decode", workloads.decode_layer(i), [workloads.decode_x(i)], 3, True))
    out.append(one("skinny", workloads.skinny_layer(), [workloads.skinny_x(2), workloads.skinny_x(32)], 3, True))
    for i, (nm, _, _) in enumerate(workloads.DECODER_BLOCK):
        out.append(one(f"block_{nm}", workloads.block_layer(i), [workloads.block_x(i)], 1, False))
    shape = workloads.LARGE_SHAPES[0]
    out.append(one("large", workloads.large_layer(shape), [workloads.large_x(shape, 1), workloads.large_x(shape, 32)],
                   1, False))
    log(f"  oracle per workload: {time.perf_counter() - t0:.1f} s")
    return {"threads": threads, "configs": out}


def traffic_entry(family):
    """HBM bytes per launch of one kernel family of the step, from the committed
    rocprofv3 --pmc summary, if it was taken on the family's current sources;
    else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    fam = t.get("families", {}).get(family)
    if not fam or fam.get("kernel_source_hash") != kernel_source_hash(family):
        return None
    return fam.get("bytes_per_launch")


def family_row(name, launches_per_step, steps, phase_ms, alg_per_step):
    """Roofline figures of one kernel family from its phase of the timed region."""
    mean_us = phase_ms * 1e3 / (steps * launches_per_step)
    alg = alg_per_step / launches_per_step
    achieved = alg / (mean_us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic_entry(name), "kernel": name,
            "mean_launch_us": round(mean_us, 3), "alg_bytes_per_launch": round(alg, 1),
            "launches": steps * launches_per_step}


def headline(steps, steps_requested, warmup, gemv_ms, skinny_ms, step, per_call, ceiling, cpu, full_path):
    """The compact result line (a few KB): everything the metric needs, nothing
    that grows with the number of sections."""
    ms = gemv_ms + skinny_ms
    value = step["bytes"] * steps / (ms * 1e-3) / 1e9
    fams = [family_row("gemv_kernel", step["gemv_launches"], steps, gemv_ms, step["gemv_bytes"]),
            family_row("pipe_kernel", step["skinny_launches"], steps, skinny_ms, step["skinny_bytes"])]
    dom = max(fams, key=lambda f: f["mean_launch_us"] * f["launches"])
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "steps_requested": steps_requested, "warmup": warmup, "ms_per_step": round(ms / steps, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "pct_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "config": {"workload": "one step = the decode GEMV at M=1 (bf16 x, zero bias; e4m3 weights [4096,4096], "
                               "[14336,4096], [4096,14336]) + the skinny sweep at M=2,4,8,16,22,32 (fp16 x, fp16 "
                               "bias; e4m3 weight [14336,4096], Student-t(3) rows); per-channel scales; weight copies "
                               "rotated through >= 1 GiB per layer",
                   "m": [1] + list(workloads.SKINNY_MS), "bytes_per_step": step["bytes"],
                   "calls_per_step": step["gemv_launches"] + step["skinny_launches"],
                   "launch": "eager, C ABI on torch's current stream"},
        "roofline": dom,
        "kernels": [{k: f[k] for k in ("kernel", "mean_launch_us", "achieved", "frac", "traffic", "launches")}
                    for f in fams],
        "per_call": per_call,
        "read_ceiling": ceiling,
        "cpu_baseline": cpu,
        "full_record": os.path.relpath(full_path, ROOT) if full_path else None,
    }


def compact_call(r):
    return {"n": r["n"], "k": r["k"], "m": r["m"], "kernel": r["kernel"], "us": r["us_per_call"],
            "pct_peak": r["pct_peak"]}


def main():
    global SPIN_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-ms", type=float, default=MIN_TIMED_MS,
                    help="shortest timed region: fewer steps than this lasts are replaced by enough steps")
    ap.add_argument("--spin-ms", type=float, default=SPIN_MS,
                    help="milliseconds of the same work run before each timed region (GPU clock ramp-up)")
    ap.add_argument("--extra", action="store_true", help="also time the other workloads (full record only)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-oracle-workloads", action="store_true",
                    help="skip timing the oracle on every workload (full record only)")
    ap.add_argument("--full-json", default=FULL_RECORD, help="where the full record is written ('' for nowhere)")
    ap.add_argument("--only-timed", action="store_true",
                    help="run only the timed region (for profiler runs: the last 9*steps library launches are it)")
    ap.add_argument("--only", choices=SECTIONS, nargs="+",
                    help="run only these extra sections (no step) and print their JSON")
    ap.add_argument("--reps", type=int, default=100, help="launches per burst in the extra sections")
    ap.add_argument("--shape", nargs=3, type=int, metavar=("N", "K", "M"),
                    help="time one fp8w_linear shape alone (N(0,0.02^2) weights, no bias, weight copies rotated "
                         "through >= 1 GiB): --steps back-to-back launches, then print its JSON (profiler runs)")
    ap.add_argument("--act", choices=("bf16", "fp16"), default="bf16", help="activation dtype of --shape")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="print a markdown table of the library's kernels in a rocprofv3 kernel trace, then exit")
    ap.add_argument("--last", type=int, default=None,
                    help="with --trace-summary: only the last N library dispatches")
    ap.add_argument("--mfma-summary", nargs=3, metavar=("PMC_CSV", "N", "K"),
                    help="print a markdown table of the skinny kernels' matrix-core counters, then exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/step_traffic.json from two rocprofv3 --pmc runs of --only-timed, then exit")
    ap.add_argument("--counter-summary", nargs="+", metavar="ARG",
                    help="KERNEL CSV [CSV ...]: mean per dispatch of every counter in rocprofv3 --pmc CSVs for the "
                         "library kernels whose name contains KERNEL, then exit")
    args = ap.parse_args()
    SPIN_MS = args.spin_ms
    if args.counter_summary:
        counter_summary(args.counter_summary[0], args.counter_summary[1:])
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], TRAFFIC_FILE)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary[0], int(args.mfma_summary[1]), int(args.mfma_summary[2]))
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.last)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (each GPU would hold its own "
              "shard of the weight; the per-GPU kernel is what is measured here)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    fw.load()
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} CUs={props.multi_processor_count} mem={props.total_memory / 2**30:.0f} GiB")

    if args.only:
        out = extra_sections(dev, stream, args.reps, args.only)
        calibration_copy(dev)
        print(json.dumps(out), flush=True)
        return

    if args.shape:
        n, k, m = args.shape
        case = workloads.random_case(7, m, n, k, torch.bfloat16 if args.act == "bf16" else torch.float16,
                                     with_bias=False)
        L = Layer(case.layer, max(1, math.ceil(ROTATE_BYTES / (n * k))), dev)
        c = Call(L, case.x.to(dev), dev)
        r = call_report(c, burst(c, args.steps, args.warmup, stream))
        calibration_copy(dev)
        print(json.dumps(r), flush=True)
        return

    # ---------------------------------------------------------------- the step (the metric)
    step = Step(dev)
    log(f"step: {step.step_bytes / 1e6:.2f} MB ({len(step.calls)} calls); rotated copies: decode "
        f"{step.dec_copies}, skinny {step.sk_copies}")
    shape = {"bytes": step.step_bytes, "gemv_launches": len(step.dec_calls),
             "skinny_launches": len(step.sk_calls), "gemv_bytes": step.dec_step_bytes,
             "skinny_bytes": step.sk_step_bytes}

    if args.only_timed:
        g_ms, s_ms = timed_region(step, args.steps, args.warmup, dev)
        calibration_copy(dev)
        line = headline(args.steps, args.steps, args.warmup, g_ms, s_ms, shape, None, None, None, None)
        print(json.dumps({k: line[k] for k in ("value", "steps", "ms_per_step", "roofline", "kernels")}),
              flush=True)
        return

    per_call, full_calls = [], []
    for c in step.calls:
        r = call_report(c, burst(c, 200, 20, stream))
        full_calls.append(r)
        per_call.append(compact_call(r))
        log(f"  {r['layer']} m={r['m']}: {r['us_per_call']:.2f} us/call  {r['gbps']:.0f} GB/s "
            f"({r['pct_peak']:.1f}% of 8 TB/s) [{r['kernel']}]")
    ceiling = read_ceiling(dev, sorted({c.layer.n * c.layer.k for c in step.calls}))

    steps = args.steps
    g_ms, s_ms = timed_region(step, steps, args.warmup, dev)
    if g_ms + s_ms < args.min_ms:
        steps = max(steps, math.ceil(args.min_ms / ((g_ms + s_ms) / steps)))
        log(f"  {args.steps} steps took {g_ms + s_ms:.2f} ms; timing {steps} steps")
        g_ms, s_ms = timed_region(step, steps, args.warmup, dev, spin=False)
    log(f"timed region: {steps} steps, {(g_ms + s_ms) * 1e3 / steps:.2f} us/step "
        f"(M=1 phase {g_ms * 1e3 / steps:.2f}, M=2..32 phase {s_ms * 1e3 / steps:.2f})")

    full = {"per_call": full_calls,
            "warm_per_call": [call_report(c, burst(c, 200, 20, stream, warm=True)) for c in step.calls],
            "host_latency": [dict(layer=c.layer.name, m=c.m, **host_latency(c, stream)) for c in step.calls],
            "read_ceiling": ceiling}
    if args.extra:
        full["extra"] = extra_sections(dev, stream, args.reps)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(step, args.cpu_budget)
        log(f"cpu baseline: {cpu['value']} GB/s on {cpu['cores']} threads, {cpu['one_core']['value']} GB/s on one; "
            f"GPU results vs this oracle run: {'pass' if cpu['gpu_parity_vs_this_oracle_run'] else 'FAIL'}")
        if not args.no_oracle_workloads:
            full["oracle_per_workload"] = oracle_per_config()

    calibration_copy(dev)
    line = headline(steps, args.steps, args.warmup, g_ms, s_ms, shape, per_call,
                    [{"bytes": c["bytes"], "us": c["us"], "pct_peak": c["pct_peak"]} for c in ceiling], cpu,
                    args.full_json or None)
    full["headline"] = line
    if args.full_json:
        os.makedirs(os.path.dirname(os.path.abspath(args.full_json)), exist_ok=True)
        with open(args.full_json, "w") as f:
            json.dump(full, f, indent=1)
    print(json.dumps(line), flush=True)


COPY_BYTES = 256 << 20


def calibration_copy(dev):
    """A plain 256 MiB device-to-device copy (torch): the known-size point that
    scales the profiler's FETCH_SIZE / WRITE_SIZE readings to bytes."""
    a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()


def _pmc_rows(path, counter):
    import csv
    with open(path) as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def counter_summary(kernel, csvs):
    """Markdown table: for the library dispatches whose name contains `kernel`,
    the mean per dispatch of every counter in the given rocprofv3 --pmc CSVs
    (one counter set per run). FETCH_SIZE and WRITE_SIZE (KiB) are also given
    in bytes, scaled by what the same run's last device copy (bench.py's 256 MiB
    calibration) reads for them."""
    import csv
    print("| Counter | Mean per dispatch | Dispatches | Bytes (calibrated) |")
    print("|---|---|---|---|")
    for path in csvs:
        with open(path) as f:
            rows = list(csv.DictReader(f))
        for name in sorted({r["Counter_Name"] for r in rows}):
            vals = [float(r["Counter_Value"]) for r in rows
                    if r["Counter_Name"] == name and kernel in r["Kernel_Name"] and "fp8w::" in r["Kernel_Name"]]
            if not vals:
                continue
            mean = sum(vals) / len(vals)
            cal = ""
            if name in ("FETCH_SIZE", "WRITE_SIZE"):
                copies = [r for r in rows if r["Counter_Name"] == name and
                          ("copyBuffer" in r["Kernel_Name"] or "direct_copy" in r["Kernel_Name"])]
                if copies:
                    copy = float(max(copies, key=lambda r: int(r["Dispatch_Id"]))["Counter_Value"])
                    cal = f"{mean * COPY_BYTES / copy / 1e6:.2f} MB"
            print(f"| {name} | {mean:,.1f} | {len(vals)} | {cal} |")


def pmc_summary(fetch_csv, write_csv, out_path):
    """Turn two rocprofv3 --pmc runs of `bench.py --only-timed` (FETCH_SIZE, then
    WRITE_SIZE, KiB per dispatch) into HBM bytes per launch of each kernel
    family of the step, each counter scaled by what it reads for the 256 MiB
    calibration copy at the end of the run."""
    res = {}
    for name, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _pmc_rows(path, name)
        # the calibration copy is the run's last and largest device copy (a blit
        # kernel or an elementwise copy, depending on how torch lowers it)
        copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"] or "direct_copy" in r["Kernel_Name"]]
        copy = float(max(copies, key=lambda r: int(r["Dispatch_Id"]))["Counter_Value"]) if copies else None
        factor = (COPY_BYTES / 1024.0) / copy if copy else None
        res[name] = {"copy_kib": copy, "scale": factor, "families": {}}
        for fam in FAMILIES:
            vals = [float(r["Counter_Value"]) for r in rows if fam in r["Kernel_Name"] and "fp8w::" in r["Kernel_Name"]]
            res[name]["families"][fam] = {"kib_mean": sum(vals) / len(vals) if vals else None,
                                          "dispatches": len(vals)}
    shapes = {"gemv_kernel": [(1, n, k, True) for n, k in workloads.DECODE_SHAPES],
              "pipe_kernel": [(m, 14336, 4096, True) for m in workloads.SKINNY_MS]}
    out = {"kernels": "the step's two kernel families, all their launches in a run of bench.py --only-timed",
           "counters": res, "families": {}}
    for fam in FAMILIES:
        f = res["FETCH_SIZE"]["families"][fam]["kib_mean"]
        w = res["WRITE_SIZE"]["families"][fam]["kib_mean"]
        if f is None or w is None:
            continue
        fetch = f * 1024 * res["FETCH_SIZE"]["scale"]
        write = w * 1024 * res["WRITE_SIZE"]["scale"]
        alg = sum(alg_bytes(*s) for s in shapes[fam]) / len(shapes[fam])
        out["families"][fam] = {"kernel_source_hash": kernel_source_hash(fam), "bytes_per_launch": round(fetch + write, 1),
                                "fetch_bytes_per_launch": round(fetch, 1), "write_bytes_per_launch": round(write, 1),
                                "alg_bytes_per_launch": alg, "traffic_over_alg": round((fetch + write) / alg, 4)}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def _short_kernel_name(full):
    """'pipe_kernel<XR=16,CT=4,KP=1,NS=4>'-style name from a demangled trace name."""
    import re
    full = full.replace("(anonymous namespace)::", "").replace("fp8w::", "")
    m = re.search(r"(\w+_kernel)(<[^()]*>)?\(", full)
    if not m:
        return full[:60]
    name, targs = m.group(1), (m.group(2) or "")
    args = [a.strip() for a in targs[1:-1].split(",")] if targs else []
    keys = {"pipe_kernel": ("XR", "CT", "KP", "NS", "CB"), "seg_kernel": ("SEG", "T", "W", "U", "MT"),
            "gemv_kernel": ("R", "U", "NT", "DB", "CH"), "gemv_shift_kernel": ("R", "U", "NT", "DB"),
            "narrow_kernel": ("MT", "W", "NS"), "wpipe_kernel": ("XR", "CT", "NS"), "w8a8_kernel": ("BN", "BM", "NS", "WN", "WM", "GM"),
            "gemv_grouped_kernel": ("R", "U", "NT", "DB"), "pipe_grouped_kernel": ("XR", "CT", "KP", "NS", "G"),
            "batch_kernel": ("BN", "BM", "WN", "WM", "G", "GM")}.get(name)
    if keys and len(args) == len(keys) + 1:  # first argument is the activation type
        short = f"{name}<" + ",".join(f"{kk}={v}" for kk, v in zip(keys, args[1:])) + ">"
        # the library's names give the load width only where it is not 16 bytes
        return short.replace(",CB=16>", ">").replace(",CH=16>", ">")
    return name + targs


def trace_summary(csv_path, last=None):
    """Markdown table of the library's kernels in a rocprofv3 --kernel-trace CSV:
    one row per kernel instance and grid (the grid identifies the shape), with
    launch count and duration statistics in microseconds. `last` keeps only the
    last `last` library dispatches (the timed region of bench.py --only-timed)."""
    import csv
    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Dispatch_Id"]))
    ours = [r for r in rows if "fp8w::" in r["Kernel_Name"]]
    if last:
        ours = ours[-last:]
    groups = {}
    for r in ours:
        name = _short_kernel_name(r["Kernel_Name"])
        wgs = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])) * int(r.get("Grid_Size_Y") or 1)
               * int(r.get("Grid_Size_Z") or 1))
        key = (name, wgs, int(r["Workgroup_Size_X"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = ["| Kernel | Workgroups x threads | Launches | Mean (us) | p10 (us) | Median (us) | p90 (us) | Min (us) |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, wgs, wg), d in groups.items():
        d = np.array(d)
        lines.append(f"| `{name}` | {wgs} x {wg} | {len(d)} | {d.mean():.3f} | {np.percentile(d, 10):.3f} | "
                     f"{np.median(d):.3f} | {np.percentile(d, 90):.3f} | {d.min():.3f} |")
    print("\n".join(lines))


def mfma_summary(csv_path, n, k):
    """Markdown table from a rocprofv3 --pmc run with the derived counters
    MfmaFlopsF16, MfmaFlopsBF16 and MfmaUtil over the skinny kernels of an
    [n, k] weight: matrix-core FLOPs each launch issued (counted) next to the
    tile formula's figure, and the share of the run's SIMD cycles the matrix
    cores were busy."""
    import csv
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if not any(t in r["Kernel_Name"] for t in ("pipe_kernel", "seg_kernel")):
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": _short_kernel_name(r["Kernel_Name"]),
                                                   "wgs": int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])),
                                                   "wg": int(r["Workgroup_Size"]), "vgpr": r["VGPR_Count"],
                                                   "lds": r["LDS_Block_Size"]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    groups = {}
    for d in per.values():
        groups.setdefault((d["name"], d["wgs"], d["wg"], d["vgpr"], d["lds"]), []).append(d)
    lines = ["| Kernel | Workgroups x threads | VGPRs | LDS (B) | Launches | Issued GFLOP / launch (counted) | "
             "Issued GFLOP (tile formula) | Padded M | MFMA busy (% of SIMD cycles) |",
             "|---|---|---|---|---|---|---|---|---|"]
    for (name, wgs, wg, vgpr, lds), ds in groups.items():
        fl = np.mean([d.get("MfmaFlopsF16", 0.0) + d.get("MfmaFlopsBF16", 0.0) for d in ds]) / 1e9
        util = np.mean([d.get("MfmaUtil", float("nan")) for d in ds])
        issued, mpad = mfma_issued_flops(name, 0, n, k)
        exp = f"{issued / 1e9:.3f}" if issued else "-"
        lines.append(f"| `{name}` | {wgs} x {wg} | {vgpr} | {lds} | {len(ds)} | {fl:.3f} | {exp} | {mpad or '-'} | "
                     f"{util:.2f} |")
    print("\n".join(lines))


SECTIONS = ("tiny", "skinny", "block", "large", "batch", "grouped", "w8a8")


def extra_sections(dev, stream, reps=100, only=None):
    ex = {}
    want = set(only or SECTIONS)

    if "tiny" in want:
        # latency-bound calls: the 1024x1024 GEMV and the pages' example shape
        # ([22,1024] x [1024,4096]), cold (rotated) and warm, plus host wall time
        tiny = []
        for case in (workloads.tiny_gemv(), workloads.pages_example()):
            n, k = case.layer.w.shape
            per = alg_bytes(case.x.shape[0], n, k, case.layer.bias is not None)
            L = Layer(case.layer, max(1, math.ceil(ROTATE_BYTES / per)), dev)
            c = Call(L, case.x.to(dev), dev)
            r = call_report(c, burst(c, 400, 20, stream))
            r["warm"] = call_report(c, burst(c, 400, 20, stream, warm=True))
            r["host"] = host_latency(c, stream)
            tiny.append(r)
            log(f"  {r['layer']} m={r['m']}: {r['us_per_call']:.2f} us cold, {r['warm']['us_per_call']:.2f} us warm, "
                f"{r['host']['call_and_sync_us']:.1f} us call+sync [{r['kernel']}]")
            del L, c
            torch.cuda.empty_cache()
        ex["tiny"] = tiny

    if "skinny" in want:
        # skinny sweep, fp16 activations
        per = alg_bytes(32, 14336, 4096)
        L = Layer(workloads.skinny_layer(), max(1, math.ceil(ROTATE_BYTES / per)), dev)
        sk = []
        for m in workloads.SKINNY_MS:
            c = Call(L, workloads.skinny_x(m).to(dev), dev)
            sk.append(call_report(c, burst(c, reps, 10, stream)))
            r = sk[-1]
            log(f"  skinny m={m}: {r['us_per_call']:.2f} us {r['pct_peak']:.1f}% of peak, MFMA useful "
                f"{r['mfma']['useful_pct_of_peak']:.2f}% / issued {r['mfma']['issued_pct_of_peak']:.2f}% "
                f"[{r['kernel']}]")
        ex["skinny_sweep"] = sk
        ex["skinny_quantize_ms"] = round(L.quantize_ms, 3)
        del L
        torch.cuda.empty_cache()

    if "block" in want:
        # one decoder block at M = 16: seven calls per step, per-call bursts, eager
        # and graph-replayed steps; then the same block with q/k/v and gate/up
        # merged into one call each (their weights concatenated along n before
        # quantization: per-row scales make the codes identical), four calls
        blk_bytes = sum(alg_bytes(16, n, k, False) for _, n, k in workloads.DECODER_BLOCK)
        copies = max(1, math.ceil(ROTATE_BYTES / blk_bytes))
        lws = [workloads.block_layer(i) for i in range(len(workloads.DECODER_BLOCK))]
        Ls = [Layer(lw, copies, dev) for lw in lws]
        calls = [Call(Li, workloads.block_x(i).to(dev), dev) for i, Li in enumerate(Ls)]
        blk = [call_report(c, burst(c, reps, 10, stream)) for c in calls]
        gsteps = copies * -(-200 // copies)  # whole passes over the weight copies
        ms = timed_steps(calls, 200, 10, copies, False, dev)
        gms = timed_steps(calls, gsteps, 10, copies, True, dev)
        ex["decoder_block"] = {"calls": blk, "us_sum_of_calls": round(sum(b["us_per_call"] for b in blk), 2),
                               "step_us": round(ms * 1e3 / 200, 2), "step_mode": "eager",
                               "step_gbps": round(blk_bytes / (ms * 1e-3 / 200) / 1e9, 1),
                               "graph_step_us": round(gms * 1e3 / gsteps, 2), "bytes": blk_bytes}
        log(f"  decoder block m=16: {ex['decoder_block']['step_us']:.1f} us/step (eager), "
            f"{ex['decoder_block']['graph_step_us']:.1f} (graph), {ex['decoder_block']['step_gbps']:.0f} GB/s")
        del Ls, calls
        torch.cuda.empty_cache()

        groups = workloads.MERGED_BLOCK
        mlws = [workloads.Linear("+".join(lws[i].name for i in g), np.concatenate([lws[i].w for i in g]), None)
                for g in groups]
        mbytes = sum(alg_bytes(16, lw.w.shape[0], lw.w.shape[1], False) for lw in mlws)
        Ms = [Layer(lw, copies, dev) for lw in mlws]
        mcalls = [Call(Mi, workloads.block_x(g[0]).to(dev), dev) for Mi, g in zip(Ms, groups)]
        mblk = [call_report(c, burst(c, reps, 10, stream)) for c in mcalls]
        ms = timed_steps(mcalls, 200, 10, copies, False, dev)
        gms = timed_steps(mcalls, gsteps, 10, copies, True, dev)
        ex["decoder_block_merged"] = {
            "calls": mblk, "us_sum_of_calls": round(sum(b["us_per_call"] for b in mblk), 2),
            "step_us": round(ms * 1e3 / 200, 2), "step_mode": "eager",
            "step_gbps": round(mbytes / (ms * 1e-3 / 200) / 1e9, 1), "graph_step_us": round(gms * 1e3 / gsteps, 2),
            "bytes": mbytes}
        log(f"  decoder block m=16, merged q/k/v and gate/up: {ex['decoder_block_merged']['step_us']:.1f} us/step "
            f"(eager), {ex['decoder_block_merged']['graph_step_us']:.1f} (graph), "
            f"{ex['decoder_block_merged']['step_gbps']:.0f} GB/s")
        del Ms, mcalls
        torch.cuda.empty_cache()

    if "grouped" in want:
        # group scales along k: the decode layers at M = 1 (bf16) and the skinny
        # layer at M = 2, 16, 32 (fp16), with g = 32 and g = 128; then the
        # decode layers at the batched-decode sizes (the batch GEMM)
        gr = []
        for g in (32, 128):
            for i in range(3):
                lw = workloads.decode_layer(i)
                n, k = lw.w.shape
                L = GroupedLayer(lw, g, max(1, math.ceil(ROTATE_BYTES / grouped_bytes(1, n, k, g, True))), dev)
                c = GroupedCall(L, workloads.decode_x(i).to(dev), dev)
                gr.append(grouped_report(c, burst(c, 200, 20, stream)))
                gr[-1]["quantize_ms"] = round(L.quantize_ms, 3)
                log(f"  grouped g={g} {L.name} m=1: {gr[-1]['us_per_call']:.2f} us {gr[-1]['pct_peak']:.1f}% "
                    f"[{c.kernel}]")
                del L, c
                torch.cuda.empty_cache()
            L = GroupedLayer(workloads.skinny_layer(), g,
                             max(1, math.ceil(ROTATE_BYTES / grouped_bytes(32, 14336, 4096, g, True))), dev)
            for m in (2, 16, 32):
                c = GroupedCall(L, workloads.skinny_x(m).to(dev), dev)
                gr.append(grouped_report(c, burst(c, reps, 10, stream)))
                log(f"  grouped g={g} skinny m={m}: {gr[-1]['us_per_call']:.2f} us {gr[-1]['pct_peak']:.1f}% "
                    f"[{c.kernel}]")
            del L
            torch.cuda.empty_cache()
        for g in (32, 128):
            for i in range(3):
                lw = workloads.decode_layer(i)
                n, k = lw.w.shape
                L = GroupedLayer(lw, g, max(1, math.ceil(ROTATE_BYTES / grouped_bytes(max(workloads.BATCH_MS), n, k,
                                                                                      g, True))), dev)
                for m in workloads.BATCH_MS:
                    c = GroupedCall(L, workloads.batch_x(i, m).to(dev), dev)
                    gr.append(grouped_report(c, burst(c, reps, 10, stream)))
                    log(f"  grouped g={g} {L.name} m={m}: {gr[-1]['us_per_call']:.2f} us "
                        f"{gr[-1]['tflops']:.0f} TFLOP/s [{c.kernel}]")
                    del c
                del L
                torch.cuda.empty_cache()
        ex["grouped"] = gr

    if "large" in want:
        # large shapes and the k = 8200 fallback
        lg = []
        for shape in workloads.LARGE_SHAPES + [workloads.LARGE_FALLBACK_SHAPE]:
            per = alg_bytes(32, *shape, False)
            L = Layer(workloads.large_layer(shape), max(1, math.ceil(ROTATE_BYTES / per)), dev)
            for m in workloads.LARGE_MS:
                x = workloads.large_x(shape, m).to(dev)
                c = Call(L, x, dev)
                lg.append(call_report(c, burst(c, max(20, reps // 2), 5, stream)))
                log(f"  large {shape} m={m} [{lg[-1]['kernel']}]: {lg[-1]['us_per_call']:.2f} us "
                    f"{lg[-1]['pct_peak']:.1f}% of peak")
                if shape == workloads.LARGE_FALLBACK_SHAPE:  # the dequantizing fallback, forced, for comparison
                    c = Call(L, x, dev, path=fw.PATH_FALLBACK)
                    lg.append(dict(call_report(c, burst(c, max(20, reps // 2), 5, stream)), forced=True))
                    log(f"  large {shape} m={m} forced [{lg[-1]['kernel']}]: {lg[-1]['us_per_call']:.2f} us "
                        f"{lg[-1]['pct_peak']:.1f}% of peak")
            lg.append({"layer": L.name, "quantize_ms": round(L.quantize_ms, 3)})
            del L
            torch.cuda.empty_cache()
        ex["large"] = lg

    if "batch" in want:
        # batched decode: the decode weights at M = 64, 128, 256 (bf16), the
        # weight-only batch GEMM (k split over workgroups where its plan asks,
        # workspace given); bytes against HBM and FLOPs against the bf16 matrix cores
        bt = []
        for i in range(len(workloads.DECODE_SHAPES)):
            lw = workloads.decode_layer(i)
            n, k = lw.w.shape
            L = Layer(lw, max(1, math.ceil(ROTATE_BYTES / (n * k))), dev)
            for m in workloads.BATCH_MS:
                c = Call(L, workloads.batch_x(i, m).to(dev), dev)
                r = call_report(c, burst(c, max(20, reps // 2), 5, stream))
                r["pct_bf16_mfma_peak"] = round(100.0 * r["tflops"] / MFMA_PEAK_TFLOPS, 2)
                bt.append(r)
                log(f"  batch {L.name} m={m}: {r['us_per_call']:.2f} us {r['gbps']:.0f} GB/s ({r['pct_peak']:.1f}% "
                    f"of 8 TB/s), {r['tflops']:.0f} TFLOP/s ({r['pct_bf16_mfma_peak']:.1f}% of 2.5 PF) [{r['kernel']}]")
                del c
            del L
            torch.cuda.empty_cache()
        ex["batch"] = bt

    if "w8a8" in want:
        # prefill: the W8A8 layer on the decoder block's three distinct shapes
        # at M = 512, 2048, 4096 (bf16), matrix-core bound; weights rotated as
        # elsewhere; the whole layer, the GEMM alone and the activation quantizer
        pf = []
        for i in range(len(workloads.PREFILL_SHAPES)):
            lw = workloads.prefill_layer(i)
            n, k = lw.w.shape
            L = Layer(lw, max(1, math.ceil(ROTATE_BYTES / (n * k))), dev)
            for m in workloads.PREFILL_MS:
                x = workloads.prefill_x(i, m).to(dev)
                for mode in ("layer", "gemm", "quantize_x"):
                    c = W8Call(L, x, dev, mode)
                    pf.append(w8a8_report(c, burst(c, max(20, reps // 2), 5, stream, spin_ms=min(SPIN_MS, 50.0))))
                    r = pf[-1]
                    if mode == "quantize_x":
                        log(f"  w8a8 {L.name} m={m} quantize x: {r['us_per_call']:.2f} us {r['gbps']:.0f} GB/s")
                    else:
                        log(f"  w8a8 {L.name} m={m} {mode}: {r['us_per_call']:.2f} us {r['tflops']:.0f} TFLOP/s "
                            f"({r['pct_fp8_peak']:.1f}% of 5.0 PF) [{r['kernel']}]")
                    del c
            del L
            torch.cuda.empty_cache()
        ex["w8a8"] = pf
    return ex


if __name__ == "__main__":
    main()
