"""bench.py's stdout line (CPU only): the headline is a compact JSON object that
carries every field the metric needs, whatever the other sections hold, so the
whole line survives a log tail of a few KB."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def _line(steps=480, requested=20):
    shape = {"bytes": 490_000_000, "gemv_launches": 3, "skinny_launches": 6, "gemv_bytes": 134_400_000,
             "skinny_bytes": 355_600_000}
    per_call = [{"n": n, "k": k, "m": m, "kernel": "pipe_kernel<XR=32,CT=4,KP=1,NS=4>x4+splitk_reduce_kernel",
                 "us": 12.345, "pct_peak": 61.23}
                for (n, k, m) in [(4096, 4096, 1), (14336, 4096, 1), (4096, 14336, 1)]
                + [(14336, 4096, m) for m in workloads.SKINNY_MS]]
    ceiling = [{"bytes": 16777216, "us": 4.06, "pct_peak": 51.7}, {"bytes": 58720256, "us": 10.16, "pct_peak": 72.2}]
    cpu = {"value": 36.2, "unit": "GB/s", "cores": 16, "kind": "oracle", "sample": "x" * 150,
           "one_core": {"value": 2.49, "unit": "GB/s", "cores": 1, "sample": "y" * 60},
           "gpu_parity_vs_this_oracle_run": True, "host_cpus": 128, "host_model": "AMD EPYC 9575F 64-Core Processor"}
    return bench.headline(steps, requested, 5, 12.0, 38.0, shape, per_call, ceiling, cpu,
                          os.path.join(ROOT, "results", "bench_full.json"))


def test_headline_is_compact_and_complete():
    line = _line()
    text = json.dumps(line)
    assert "\n" not in text
    assert len(text) < 6000, len(text)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["metric"] == "fp8-weight linear achieved HBM GB/s (% of peak) + µs/call, M=1..32, K,N=4096..8192"
    assert line["n_gpus"] == 1 and line["steps"] == 480 and line["steps_requested"] == 20
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in line["roofline"], key
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] == 16
    assert "workload" in line["config"]


def test_headline_arithmetic():
    """value = bytes of the timed steps / their time; each family's achieved =
    its bytes per launch / its mean launch time; the roofline is the family with
    the larger share of the time."""
    line = _line()
    ms = 12.0 + 38.0
    assert abs(line["value"] - 490_000_000 * 480 / (ms * 1e-3) / 1e9) < 0.1
    assert abs(line["ms_per_step"] - ms / 480) < 1e-6
    gemv, pipe = line["kernels"]
    assert gemv["kernel"] == "gemv_kernel" and pipe["kernel"] == "pipe_kernel"
    assert abs(gemv["mean_launch_us"] - 12.0e3 / (480 * 3)) < 1e-3
    assert abs(pipe["achieved"] - (355_600_000 / 6) / (38.0e-3 / (480 * 6)) / 1e9) < 0.2
    assert line["roofline"]["kernel"] == "pipe_kernel"
    assert abs(line["roofline"]["frac"] - pipe["achieved"] / 8000.0) < 1e-4
