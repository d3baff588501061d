"""The per-call entry points recorded into a HIP graph and replayed.

Every path enqueues only kernel launches with the caller's buffers (no
allocation, no memset, no host copy), so a captured sequence must replay to
the eager results, bit for bit: each call is deterministic. The graph holds a
GEMV, a single-pass and a split-k skinny call, a split and a single-pass call
of the batch GEMM, a fallback call, grouped calls (skinny and batch) and a W8A8 layer. Between replays the outputs are overwritten with NaN and
unrelated eager calls run on the same stream, so a replay that skipped a
launch or read a stale buffer would show.
"""
import pytest
import torch

import fp8_weight_only_amd as fw
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# (kind, m, n, k, dtype, kernel the dispatcher must pick, or None)
CALLS = [
    ("linear", 1, 1000, 1024, torch.bfloat16, "gemv_kernel<R=2,U=2,NT=64,DB>"),
    ("linear", 8, 2048, 1024, torch.float16, None),
    ("linear", 20, 4100, 10240, torch.bfloat16, "pipe_kernel<XR=24,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"),
    ("linear", 12, 2000, 4096, torch.float16, "narrow_kernel<MT=1,W=8,NS=2,QL>"),
    ("linear", 3, 300, 1004, torch.bfloat16, None),  # k % 8 != 0: fallback through the workspace
    ("linear", 5, 700, 2056, torch.float16, "pipe_kernel<XR=8,CT=1,KP=2,NS=4,CB=8>"),  # shifted rows, k tail
    ("linear", 1, 900, 1032, torch.bfloat16, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),  # rows of alternating alignment
    ("linear", 70, 640, 1024, torch.float16, "batch_kernel<BN=32,BM=32,W=1>x2+splitk_reduce_kernel"),
    ("linear", 300, 2048, 512, torch.bfloat16, "batch_kernel<BN=64,BM=32,W=2>"),
    ("grouped32", 1, 512, 1024, torch.bfloat16, None),
    ("grouped128", 16, 1024, 2048, torch.float16, None),
    ("grouped64", 100, 1000, 1024, torch.bfloat16, None),  # the batch GEMM with group scales, k split
    ("grouped128", 300, 2048, 512, torch.float16, None),  # and single pass
    ("w8a8", 300, 512, 512, torch.bfloat16, None),
]


class Recorded:
    """One call with its own output (and workspace) buffers, allocated before capture."""

    def __init__(self, idx, kind, m, n, k, dtype, kernel):
        case = workloads.random_case(700 + idx, m, n, k, dtype)
        self.kind = kind
        self.x = case.x.to(DEV)
        w = torch.from_numpy(case.layer.w).to(DEV)
        self.bias = case.layer.bias.to(DEV)
        if kind.startswith("grouped"):
            self.q, self.scale = fw.quantize_grouped(w, int(kind[len("grouped"):]))
            need = fw.grouped_workspace_bytes(self.x, self.q, self.scale)
            self.ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
        else:
            self.q, self.scale = fw.quantize(w)
        self.y = torch.empty((m, n), dtype=dtype, device=DEV)
        if not kind.startswith("grouped"):
            self.ws = None
        if kind == "linear":
            need = fw.workspace_bytes(self.x, self.q, self.y)
            if kernel is not None:
                path = fw.linear_path(self.x, self.q, self.y)
                name = fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, fw._dtype_code(dtype), self.x.data_ptr(),
                                             self.q.data_ptr())
                assert name == kernel, (name, kernel, path)
            if need:
                self.ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
        elif kind == "w8a8":
            self.ws = torch.empty((fw.fp8w_linear_w8a8_workspace_bytes(m, k),), dtype=torch.uint8, device=DEV)

    def run(self, out):
        if self.kind == "linear":
            fw.linear(self.x, self.q, self.scale, self.bias, out=out,
                      workspace=self.ws if self.ws is not None else torch.empty(0, dtype=torch.uint8, device=DEV))
        elif self.kind.startswith("grouped"):
            fw.linear_grouped(self.x, self.q, self.scale, self.bias, out=out, workspace=self.ws)
        else:
            fw.linear_w8a8(self.x, self.q, self.scale, self.bias, out=out, workspace=self.ws)


def test_graph_replays_match_eager():
    calls = [Recorded(i, *c) for i, c in enumerate(CALLS)]
    eager = []
    for c in calls:
        c.run(c.y)
        eager.append(c.y.clone())
    torch.cuda.synchronize()

    outs = [torch.empty_like(c.y) for c in calls]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c, o in zip(calls, outs):
            c.run(o)
    torch.cuda.synchronize()

    other = calls[1]
    scratch = torch.empty_like(other.y)
    for rep in range(3):
        print(f"replay {rep}", flush=True)
        for o in outs:
            o.fill_(float("nan"))
        other.run(scratch)  # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}, call {i} ({CALLS[i]})"
        assert torch.equal(scratch.view(torch.int16), eager[1].view(torch.int16))


def test_graph_of_several_steps_rotates_weights():
    """A graph holding several steps, each on its own weight copy (what the
    benchmark records): every step's output matches its eager call."""
    copies = 3
    base = [Recorded(20 + i, "linear", 1, 2048, 1024, torch.bfloat16, None) for i in range(copies)]
    eager = []
    for c in base:
        c.run(c.y)
        eager.append(c.y.clone())
    torch.cuda.synchronize()
    outs = [torch.empty_like(c.y) for c in base]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c, o in zip(base, outs):
            c.run(o)
    for rep in range(2):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {rep}, step {i}"
