"""Benchmark of the FP8 (e4m3) weight-only linear layer on one MI355X.

One step = one pass of the per-call hot path over the decode GEMV workload:
three fp8w_linear calls at M = 1 (bf16 activations) on the weight shapes
[4096, 4096], [14336, 4096] and [4096, 14336], each weight quantized once at
build time (that build-time quantize is timed separately). Inputs are already
resident in HBM when the timed region starts. Every step reads a different
copy of the weight codes and scales (rotating through >= 1 GiB) so the 256 MB
Infinity Cache cannot serve repeats: the kernels stream from HBM.

value = algorithmic bytes of the timed steps / timed wall time, in GB/s.
Algorithmic bytes per call = N*K (codes) + 4N (scales) + 2N (bias) + 2MK (x)
+ 2MN (y).

The roofline entry is for the dominant kernel (the M=1 GEMV): achieved =
algorithmic bytes of its launches / the sum of their durations, each launch
timed with HIP events recorded on the stream it runs on (torch's current
stream, which is the stream handed to fp8w_linear).

Also reported (in "extra"): the build-time quantize, the skinny sweep
(M = 2..32), one decoder block at M=16, the large shapes and their fallback,
each with the same MALL rotation, and the oracle on the host cores
("cpu_baseline").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
Prints ONE JSON line on stdout; progress goes to stderr.
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
PEAK_HBM_GBPS = 8000.0
ROTATE_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_decode_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(m, n, k, bias=True):
    return n * k + 4 * n + (2 * n if bias else 0) + 2 * m * k + 2 * m * n


def kernel_source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "fp8_weight_only_amd", "csrc"))):
        with open(os.path.join(ROOT, "fp8_weight_only_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


class Layer:
    """One quantized layer on the GPU with `copies` rotated copies of (q, scale)."""

    def __init__(self, lw, copies, dev, dtype=torch.bfloat16):
        w = torch.from_numpy(lw.w).to(dev)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        q, s = fw.quantize(w)
        t1.record()
        torch.cuda.synchronize()
        self.quantize_ms = t0.elapsed_time(t1)
        self.n, self.k = lw.w.shape
        self.name = lw.name
        del w
        self.qs = [(q, s)] + [(q.clone(), s.clone()) for _ in range(copies - 1)]
        self.bias = None if lw.bias is None else lw.bias.to(dev)
        self.dtype = dtype


def run_calls(calls, steps, stream, events=None):
    """calls: list of (fn_args) for fw raw linear; each step issues every call once
    with the copy index rotating. events: optional list to receive (start, end, idx)."""
    lib = fw.load()
    f = lib.fp8w_linear
    for st in range(steps):
        for ci, c in enumerate(calls):
            args = c[st % len(c)]
            if events is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                r = f(*args, stream)
                e1.record()
                events.append((e0, e1, ci))
            else:
                r = f(*args, stream)
            if r != 0:
                raise fw.Fp8wError(r, "fp8w_linear")


def build_calls(layer, x, y, ws=None):
    act = fw.BF16 if x.dtype == torch.bfloat16 else fw.FP16
    m, k = x.shape
    out = []
    for q, s in layer.qs:
        out.append((x.data_ptr(), act, m, k, q.data_ptr(), s.data_ptr(),
                    0 if layer.bias is None else layer.bias.data_ptr(), layer.n, y.data_ptr(),
                    0 if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel()))
    return out


def time_calls(calls, steps, warmup, stream):
    """Whole-step wall time (events around the timed region) and per-launch event durations."""
    run_calls(calls, warmup, stream)
    torch.cuda.synchronize()
    ev = []
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    g0.record()
    run_calls(calls, steps, stream, events=ev)
    g1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    total_ms = g0.elapsed_time(g1)
    per = [[] for _ in calls]
    for e0, e1, ci in ev:
        per[ci].append(e0.elapsed_time(e1) * 1e3)  # us
    return total_ms, wall, per


def summarize_us(v):
    a = np.asarray(v)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "mean": float(a.mean())}


def bench_shapes(name, layers, xs, steps, warmup, dev, stream, ws_bytes=0):
    ys = [torch.empty((x.shape[0], L.n), dtype=x.dtype, device=dev) for L, x in zip(layers, xs)]
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev) if ws_bytes else None
    calls = [build_calls(L, x, y, ws) for L, x, y in zip(layers, xs, ys)]
    total_ms, wall, per = time_calls(calls, steps, warmup, stream)
    rows = []
    for L, x, p in zip(layers, xs, per):
        m = x.shape[0]
        b = alg_bytes(m, L.n, L.k, L.bias is not None)
        s = summarize_us(p)
        rows.append({"layer": L.name, "m": m, "n": L.n, "k": L.k,
                     "path": ["gemv", "skinny", "fallback"][fw.linear_path(x, L.qs[0][0])],
                     "us_per_call": s, "alg_bytes": b,
                     "gbps_median": b / (s["median"] * 1e-6) / 1e9,
                     "pct_peak_median": 100.0 * b / (s["median"] * 1e-6) / 1e9 / PEAK_HBM_GBPS,
                     "tflops_median": 2.0 * m * L.n * L.k / (s["median"] * 1e-6) / 1e12})
    return {"name": name, "steps": steps, "timed_ms": total_ms, "wall_s": wall, "calls": rows}


def cpu_info():
    model = ""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                model = line.split(":", 1)[1].strip()
    except Exception:
        pass
    return os.cpu_count(), model


def cpu_baseline(layers_np, xs, budget_s=10.0):
    """The oracle (fp64 C, OpenMP over rows) on the host cores, on the same decode
    calls, repeated until ~budget_s of CPU work: GB/s of algorithmic bytes."""
    import oracle
    prepared = []
    for lw, x in zip(layers_np, xs):
        q, s, st = oracle.quantize_rows(lw.w)
        prepared.append((x.double().numpy(), q, s, None if lw.bias is None else lw.bias.double().numpy()))
    reps = 0
    byts = 0
    t0 = time.perf_counter()
    while True:
        for (x64, q, s, b), lw in zip(prepared, layers_np):
            oracle.linear_f64(x64, q, s, b)
            byts += alg_bytes(x64.shape[0], q.shape[0], q.shape[1], b is not None)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    nproc, model = cpu_info()
    return {"value": byts / el / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{reps} passes over the 3 decode GEMV calls (M=1; 4096x4096, 14336x4096, 4096x14336), "
                      f"fp64 oracle, {el:.1f} s",
            "host_cpus": nproc, "host_model": model}


def traffic_entry(bytes_per_launch):
    """HBM traffic of the GEMV from the committed rocprofv3 --pmc summary, if it was
    taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--quick", action="store_true", help="decode workload only (no extra sections)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the per-GPU shard is the "
              "measured unit; see the sharding notes in DESIGN.md)", file=sys.stderr)
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

    # ---------------------------------------------------------------- decode workload (the metric)
    per_step = sum(alg_bytes(1, n, k) for n, k in workloads.DECODE_SHAPES)
    copies = max(1, math.ceil(ROTATE_BYTES / per_step))
    log(f"decode workload: {per_step / 1e6:.2f} MB per step, {copies} rotated copies")
    lws = [workloads.decode_layer(i) for i in range(3)]
    layers = [Layer(lw, copies, dev) for lw in lws]
    xs_cpu = [workloads.decode_x(i) for i in range(3)]
    xs = [x.to(dev) for x in xs_cpu]
    quant = [{"layer": L.name, "ms": L.quantize_ms, "gbps": 5.0 * L.n * L.k / (L.quantize_ms * 1e-3) / 1e9}
             for L in layers]

    # parity of what is timed (the oracle is test infrastructure; checked once, before timing)
    parity = True
    try:
        import oracle
        for L, lw, xc, x in zip(layers, lws, xs_cpu, xs):
            q_ref, s_ref, _ = oracle.quantize_rows(lw.w)
            if not np.array_equal(L.qs[0][0].cpu().numpy(), q_ref):
                parity = False
            y = fw.linear(x, L.qs[0][0], L.qs[0][1], L.bias)
            x64 = xc.double().numpy()
            y_ref = oracle.linear_f64(x64, q_ref, s_ref, lw.bias.double().numpy())
            tol = 1e-2 * np.abs(y_ref) + 1e-3 * np.linalg.norm(x64) * oracle.row_amax(lw.w)[None, :]
            yv = y.double().cpu().numpy()
            parity &= bool(np.all(np.isfinite(yv)) and np.all(np.abs(yv - y_ref) <= tol))
    except Exception as e:  # noqa: BLE001
        log(f"parity check skipped: {e}")
        parity = None
    log(f"parity vs oracle: {parity}")

    res = bench_shapes("decode", layers, xs, args.steps, args.warmup, dev, stream)
    step_bytes = per_step
    value = step_bytes * args.steps / (res["timed_ms"] * 1e-3) / 1e9
    ms_per_step = res["timed_ms"] / args.steps
    # roofline: the GEMV launches, timed one by one with events on their stream
    gemv_bytes = sum(c["alg_bytes"] for c in res["calls"])
    gemv_us = sum(c["us_per_call"]["mean"] for c in res["calls"])
    achieved = gemv_bytes / (gemv_us * 1e-6) / 1e9
    for c in res["calls"]:
        log(f"  {c['layer']}: median {c['us_per_call']['median']:.2f} us  {c['gbps_median']:.0f} GB/s "
            f"({c['pct_peak_median']:.1f}% of 8 TB/s)")
    log(f"step: {ms_per_step * 1e3:.2f} us, {value:.0f} GB/s whole-step")

    traffic = traffic_entry(gemv_bytes / len(res["calls"]))
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "decode GEMV, M=1: three fp8w_linear calls per step on W e4m3 [4096,4096], "
                               "[14336,4096], [4096,14336] (N(0,0.02^2) weights, per-channel scales), "
                               "x bf16 N(0,1), zero bf16 bias, weights rotated through >= 1 GiB",
                   "m": 1, "shapes_nk": workloads.DECODE_SHAPES, "act_dtype": "bf16", "weight_dtype": "e4m3fn",
                   "accumulate": "f32", "rotated_copies": copies, "bytes_per_step": step_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                     "kernel": "gemv_kernel (M=1 GEMV)",
                     "alg_bytes_per_launch": gemv_bytes / len(res["calls"]),
                     "mean_launch_us": gemv_us / len(res["calls"])},
        "parity": parity,
        "per_call": res["calls"],
        "quantize": quant,
    }

    if not args.quick:
        out["extra"] = extra_sections(dev, stream, max(50, args.steps // 5), max(10, args.warmup // 5))

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)...")
        out["cpu_baseline"] = cpu_baseline(lws, xs_cpu, args.cpu_budget)
    else:
        out["cpu_baseline"] = None

    # a plain 256 MiB device copy: the calibration point for --pmc FETCH_SIZE / WRITE_SIZE
    a = torch.empty(64 << 20, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps(out), flush=True)


def extra_sections(dev, stream, steps, warmup):
    ex = {}
    # skinny sweep, fp16
    lw = workloads.skinny_layer()
    per = alg_bytes(32, 14336, 4096)
    L = Layer(lw, max(1, math.ceil(ROTATE_BYTES / per)), dev, torch.float16)
    sk = []
    for m in workloads.SKINNY_MS:
        x = workloads.skinny_x(m).to(dev)
        r = bench_shapes(f"skinny_m{m}", [L], [x], steps, warmup, dev, stream)
        c = r["calls"][0]
        log(f"  skinny m={m}: {c['us_per_call']['median']:.2f} us {c['pct_peak_median']:.1f}% of peak")
        sk.append(c)
    ex["skinny_sweep"] = sk
    ex["skinny_quantize_ms"] = L.quantize_ms
    del L
    torch.cuda.empty_cache()

    # decoder block at M=16 (seven calls per step)
    blk_bytes = sum(alg_bytes(16, n, k, False) for _, n, k in workloads.DECODER_BLOCK)
    copies = max(1, math.ceil(ROTATE_BYTES / blk_bytes))
    Ls = [Layer(workloads.block_layer(i), copies, dev) for i in range(len(workloads.DECODER_BLOCK))]
    xs = [workloads.block_x(i).to(dev) for i in range(len(workloads.DECODER_BLOCK))]
    r = bench_shapes("decoder_block_m16", Ls, xs, steps, warmup, dev, stream)
    tot_us = sum(c["us_per_call"]["median"] for c in r["calls"])
    r["block_us_sum_of_medians"] = tot_us
    r["block_gbps"] = blk_bytes / (tot_us * 1e-6) / 1e9
    r["block_step_us"] = r["timed_ms"] * 1e3 / steps
    log(f"  decoder block m=16: {tot_us:.1f} us (sum of medians), {r['block_gbps']:.0f} GB/s")
    ex["decoder_block"] = r
    del Ls
    torch.cuda.empty_cache()

    # large shapes (+ the K=8200 fallback)
    lg = []
    for shape in workloads.LARGE_SHAPES + [workloads.LARGE_FALLBACK_SHAPE]:
        lw = workloads.large_layer(shape)
        per = alg_bytes(32, *shape, False)
        L = Layer(lw, max(1, math.ceil(ROTATE_BYTES / per)), dev)
        del lw
        for m in workloads.LARGE_MS:
            x = workloads.large_x(shape, m).to(dev)
            ws = fw.workspace_bytes(x, L.qs[0][0])
            r = bench_shapes(f"large_{shape}_m{m}", [L], [x], max(20, steps // 2), warmup, dev, stream, ws)
            c = r["calls"][0]
            log(f"  large {shape} m={m} [{c['path']}]: {c['us_per_call']['median']:.2f} us "
                f"{c['pct_peak_median']:.1f}% of peak")
            lg.append(c)
        lg.append({"layer": L.name, "quantize_ms": L.quantize_ms})
        del L
        torch.cuda.empty_cache()
    ex["large"] = lg
    return ex


if __name__ == "__main__":
    main()
