"""GPU parity of the batch path (fp8w_linear above 32 tokens): the GEMM that
decodes the codes in its main loop, against the oracle's fp64 layer.

Source: "FP8 weight-only (precision: fp8_weights)", section "The contract" (the
same contract as every path: e4m3 weights, fp32 accumulation, the scale and
bias in the fp32 epilogue, one rounding to the activation dtype). Covered:
every tile shape of the kernel, each with ragged channel and token tails,
bf16 and fp16, bias and none, the shortest ring (k = 256) and k stagger over
the XCDs (k = 768 and up), and the decode layers at 64-256 tokens on sampled
outputs.
"""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_gate, assert_same_bits, gate_sampled, nan_like, oracle_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _act(dtype):
    return fw.BF16 if dtype == torch.bfloat16 else fw.FP16


TILES = [
    # (m, n, k, dtype, bias, plan the dispatcher must pick): every tile shape,
    # single pass and with k split over workgroups, ragged channel and token tails
    (33, 64, 256, torch.bfloat16, True, "batch_kernel<BN=32,BM=32,W=1>"),
    (33, 64, 1024, torch.float16, False, "batch_kernel<BN=32,BM=32,W=1>x2+splitk_reduce_kernel"),
    (33, 5000, 256, torch.bfloat16, True, "batch_kernel<BN=64,BM=32,W=2>"),
    (33, 1000, 3072, torch.float16, True, "batch_kernel<BN=64,BM=32,W=2>x6+splitk_reduce_kernel"),
    (33, 14300, 256, torch.bfloat16, False, "batch_kernel<BN=64,BM=64,W=4>"),
    (33, 3000, 2048, torch.float16, True, "batch_kernel<BN=64,BM=64,W=4>x4+splitk_reduce_kernel"),
    (70, 10000, 256, torch.bfloat16, True, "batch_kernel<BN=128,BM=64,W=8>"),
    (33, 5000, 2048, torch.float16, False, "batch_kernel<BN=128,BM=64,W=8>x4+splitk_reduce_kernel"),
    (200, 10000, 256, torch.bfloat16, True, "batch_kernel<BN=128,BM=128,W=8>"),
    (70, 10000, 3072, torch.float16, True, "batch_kernel<BN=128,BM=128,W=8>x3+splitk_reduce_kernel"),
    (257, 11264, 1024, torch.bfloat16, False, "batch_kernel<BN=256,BM=64,W=8>"),
    (33, 9216, 5120, torch.float16, True, "batch_kernel<BN=256,BM=64,W=8>x5+splitk_reduce_kernel"),
    (400, 10000, 256, torch.bfloat16, True, "batch_kernel<BN=256,BM=128,W=8>"),
    (65, 8704, 5120, torch.float16, False, "batch_kernel<BN=256,BM=128,W=8>x5+splitk_reduce_kernel"),
    (1000, 7000, 768, torch.bfloat16, True, "batch_kernel<BN=256,BM=128,W=8>"),
]


@pytest.mark.parametrize("m,n,k,dtype,bias,kernel", TILES)
def test_batch_tiles_parity(m, n, k, dtype, bias, kernel):
    print(f"batch m={m} n={n} k={k} {dtype} bias={bias} {kernel}", flush=True)
    assert fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, _act(dtype), 0, 0) == kernel
    case = workloads.random_case(900 + m + n + k, m, n, k, dtype, with_bias=bias)
    w = torch.from_numpy(case.layer.w).to(DEV)
    q, s = fw.quantize(w)
    x = case.x.to(DEV)
    b = None if case.layer.bias is None else case.layer.bias.to(DEV)
    assert fw.linear_path(x, q) == fw.PATH_BATCH
    split = "splitk" in kernel
    assert (fw.workspace_bytes(x, q) > 0) == split
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    assert_same_bits(q.cpu().numpy(), q_ref, "codes")
    y = nan_like((m, n), dtype, DEV)
    fw.linear(x, q, s, b, out=y)  # allocates the workspace a split plan asks for
    torch.cuda.synchronize()
    yv = y.double().cpu().numpy()
    assert_gate(yv, y_ref, x64, amax, kernel)
    if split:
        # no workspace: the single-pass plan, also within the gate and within
        # fp32 summation-order rounding of the split result
        y1 = nan_like((m, n), dtype, DEV)
        fw.linear(x, q, s, b, out=y1, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
        torch.cuda.synchronize()
        y1v = y1.double().cpu().numpy()
        assert_gate(y1v, y_ref, x64, amax, kernel + " single pass")
        assert np.allclose(y1v, yv, rtol=2e-2, atol=1e-2)


@pytest.mark.parametrize("m", [64, 128, 256])
def test_batch_decode_layers_sampled(m):
    """The decode step's three layers (bf16, no bias) at m tokens, every code
    bit-exact and 48 seeded output rows (all their channels) against the oracle."""
    for i, (n, k) in enumerate(workloads.DECODE_SHAPES):
        lay = workloads.decode_layer(i)
        x_cpu = workloads.activations(60 + i, m, m, k, torch.bfloat16)
        print(f"batch decode layer {n}x{k} m={m} {fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, fw.BF16, 0, 0)}",
              flush=True)
        q, s = fw.quantize(torch.from_numpy(lay.w).to(DEV))
        q_ref, s_ref, st = oracle.quantize_rows(lay.w)
        assert st == 0
        assert_same_bits(q.cpu().numpy(), q_ref, "codes")
        x = x_cpu.to(DEV)
        assert fw.linear_path(x, q) == fw.PATH_BATCH
        y = nan_like((m, n), torch.bfloat16, DEV)
        fw.linear(x, q, s, None, out=y)
        torch.cuda.synchronize()
        g = np.random.default_rng(m * 10 + i)
        rows = np.sort(g.choice(m, size=min(48, m), replace=False))
        x64 = x_cpu.double().numpy()
        cols = np.arange(n)
        rr, cc = np.meshgrid(rows, cols, indexing="ij")
        ref = oracle.linear_f64_sampled(x64, q_ref, s_ref, None, rr.ravel(), cc.ravel()).reshape(rr.shape)
        yv = y.double().cpu().numpy()[rows]
        xnorm = np.linalg.norm(x64[rows], axis=1)[:, None]
        ok = gate_sampled(yv, ref, xnorm, oracle.row_amax(lay.w)[None, :])
        assert ok.all(), f"{n}x{k} m={m}: {int((~ok).sum())} sampled outputs outside the gate"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_batch_matches_the_other_paths(dtype):
    """The same call through the batch GEMM, the skinny kernel (m <= 32) and the
    fallback: each within the gate, and within fp32 summation-order rounding of
    one another."""
    m, n, k = 32, 640, 1536
    case = workloads.random_case(77, m, n, k, dtype, with_bias=True)
    w = torch.from_numpy(case.layer.w).to(DEV)
    q, s = fw.quantize(w)
    x, b = case.x.to(DEV), case.layer.bias.to(DEV)
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    outs = []
    for p in (fw.PATH_BATCH, fw.PATH_SKINNY, fw.PATH_FALLBACK):
        y = nan_like((m, n), dtype, DEV)
        fw.linear(x, q, s, b, out=y, path=p)
        torch.cuda.synchronize()
        yv = y.double().cpu().numpy()
        assert_gate(yv, y_ref, x64, amax, f"path {p}")
        outs.append(yv)
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=2e-2, atol=1e-2)


def test_batch_is_deterministic_and_writes_only_y():
    m, n, k = 128, 4096, 4096  # a split plan: one workspace, reused without clearing
    case = workloads.random_case(78, m, n, k, torch.bfloat16, with_bias=True)
    q, s = fw.quantize(torch.from_numpy(case.layer.w).to(DEV))
    x, b = case.x.to(DEV), case.layer.bias.to(DEV)
    assert "splitk" in fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, fw.BF16, 0, 0)
    ws = torch.empty((fw.workspace_bytes(x, q),), dtype=torch.uint8, device=DEV)
    # y inside a larger buffer: the guard bands on both sides must stay untouched
    buf = torch.full((m * n + 2 * 4096,), 7.0, dtype=torch.bfloat16, device=DEV)
    y = buf[4096:4096 + m * n].view(m, n)
    fw.linear(x, q, s, b, out=y, workspace=ws)
    first = y.clone()
    for _ in range(3):
        fw.linear(x, q, s, b, out=y, workspace=ws)
        assert torch.equal(y.view(torch.int16), first.view(torch.int16))
    torch.cuda.synchronize()
    assert torch.all(buf[:4096] == 7.0) and torch.all(buf[4096 + m * n:] == 7.0)


def test_batch_zero_token_rows_give_bias():
    m, n, k = 70, 500, 512
    case = workloads.random_case(79, m, n, k, torch.float16, with_bias=True)
    xz = case.x.clone()
    xz[[0, 33, 69]] = 0.0
    q, s = fw.quantize(torch.from_numpy(case.layer.w).to(DEV))
    y = fw.linear(xz.to(DEV), q, s, case.layer.bias.to(DEV))
    torch.cuda.synchronize()
    for r in (0, 33, 69):
        assert torch.equal(y[r].cpu(), case.layer.bias)
