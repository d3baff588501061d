"""GPU parity of group-wise weight scales along k (fp8w_quantize_grouped,
fp8w_linear_grouped and its kernels, fp8w_dequantize_grouped) against the
oracle: scales and codes bit-identical, outputs within the gate.

Sources: "B04 - Precision & Quantization", sections "Post-training
quantization versus quantization-aware training" (one scale per run of g =
32 / 64 / 128 weights of a row) and "The one that matters: quantization is a
quality decision"; the Day-98 lab page's "one scale per 32" census; "FP8
weight-only (precision: fp8_weights)", section "The contract" for everything
else.
"""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_gate, assert_same_bits, nan_like

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _weights(seed, n, k, g):
    """Gaussian rows whose groups span 1e-2 .. 1e2 in magnitude (still finite in
    fp16), with one 50x outlier per row, a zero group and a row that
    underflows to scale 0."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k)).astype(np.float32)
    w *= (np.float32(10.0) ** rng.uniform(-2, 2, (n, k // g)).astype(np.float32)).repeat(g, axis=1)
    w[np.arange(n), rng.integers(0, k, n)] *= 50.0
    if n > 3 and k >= 2 * g:
        w[1, g:2 * g] = 0.0
        w[3, :] = 1e-44
    return w


@pytest.mark.parametrize("g", [32, 64, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_quantize_grouped_bit_exact(g, dtype):
    n, k = 67, 1024 + 2 * g
    w = _weights(g + 1, n, k, g)
    wt = torch.from_numpy(w).to(dtype)
    w_exact = wt.float().numpy()
    q, s = fw.quantize_grouped(wt.to(DEV), g)
    q_ref, s_ref, st = oracle.quantize_groups(w_exact, g)
    assert st == 0
    assert_same_bits(s.cpu().numpy(), s_ref, f"scales g={g} {dtype}")
    assert_same_bits(q.cpu().numpy(), q_ref, f"codes g={g} {dtype}")


@pytest.mark.parametrize("g", [32, 128])
def test_quantize_grouped_unaligned_weight_takes_the_scalar_path(g):
    n, k = 9, 4 * g
    w = _weights(7, n, k, g)
    buf = torch.empty(n * k + 1, dtype=torch.float32, device=DEV)
    wv = buf[1:].view(n, k)  # 4-byte aligned, not 16-byte aligned
    wv.copy_(torch.from_numpy(w).to(DEV))
    q, s = fw.quantize_grouped(wv, g)
    q_ref, s_ref, _ = oracle.quantize_groups(w, g)
    assert_same_bits(s.cpu().numpy(), s_ref, "scales")
    assert_same_bits(q.cpu().numpy(), q_ref, "codes")


def test_quantize_grouped_rejects_nonfinite():
    w = torch.ones((4, 256), device=DEV)
    w[2, 100] = float("nan")
    with pytest.raises(fw.Fp8wError) as e:
        fw.quantize_grouped(w, 64)
    assert e.value.status == 3


def _case(seed, m, n, k, g, dtype, bias):
    w = _weights(seed, n, k, g)
    x = workloads.activations(200 + seed, 0, m, k, dtype)
    b = workloads.to_act(np.random.default_rng(seed).standard_normal(n).astype(np.float32) * 0.1, dtype) \
        if bias else None
    return w, x, b


def _run_and_check(w, x, b, g, path, expect_kernel=None, x_offset=0, workspace=None):
    m, k = x.shape
    n = w.shape[0]
    q, s = fw.quantize_grouped(torch.from_numpy(w).to(DEV), g)
    q_ref, s_ref, _ = oracle.quantize_groups(w, g)
    assert_same_bits(q.cpu().numpy(), q_ref, "codes")
    act = fw.BF16 if x.dtype == torch.bfloat16 else fw.FP16
    if x_offset:
        buf = torch.empty(m * k + x_offset, dtype=x.dtype, device=DEV)
        xd = buf[x_offset:].view(m, k)
        xd.copy_(x.to(DEV))
    else:
        xd = x.to(DEV)
    if expect_kernel is not None:
        got = fw.fp8w_linear_grouped_kernel(path, m, n, k, g, act, xd.data_ptr(), q.data_ptr())
        assert got == expect_kernel, got
    bd = None if b is None else b.to(DEV)
    y = nan_like((m, n), x.dtype, DEV)
    fw.linear_grouped(xd, q, s, bd, out=y, path=path, workspace=workspace)
    torch.cuda.synchronize()
    x64 = x.double().numpy()
    b64 = None if b is None else b.double().numpy()
    y_ref = oracle.linear_f64_groups(x64, q_ref, s_ref, g, b64)
    assert_gate(y.double().cpu().numpy(), y_ref, x64, oracle.row_amax(w), f"m={m} n={n} k={k} g={g} path={path}")
    return y


GEMV = [
    # (n, k, g, dtype, bias)
    (1000, 1024, 32, torch.bfloat16, True),
    (37, 4352, 64, torch.float16, False),     # tail passes
    (300, 14336, 128, torch.bfloat16, True),
    (4096, 256, 32, torch.float16, True),
]


@pytest.mark.parametrize("n,k,g,dtype,bias", GEMV)
def test_grouped_gemv(n, k, g, dtype, bias):
    print(f"grouped gemv n={n} k={k} g={g}", flush=True)
    w, x, b = _case(n + k, 1, n, k, g, dtype, bias)
    _run_and_check(w, x, b, g, fw.PATH_AUTO, "gemv_grouped_kernel<R=2,U=2,NT=64,DB>")


SKINNY = [
    # (m, n, k, g, dtype, bias, kernel)
    (2, 8200, 1024, 32, torch.bfloat16, True, "pipe_grouped_kernel<XR=4,CT=4,KP=1,NS=4>"),
    (5, 16400, 512, 64, torch.float16, False, "pipe_grouped_kernel<XR=8,CT=4,KP=1,NS=2>"),
    (16, 9000, 2048, 128, torch.bfloat16, True, "pipe_grouped_kernel<XR=16,CT=4,KP=1,NS=4>"),
    (32, 8192, 1024, 32, torch.float16, True, "pipe_grouped_kernel<XR=32,CT=4,KP=1,NS=4>"),
    (22, 20000, 1536, 64, torch.bfloat16, False, "pipe_grouped_kernel<XR=32,CT=4,KP=1,NS=2>"),
    (3, 300, 2048, 32, torch.bfloat16, True, "pipe_grouped_kernel<XR=4,CT=1,KP=2,NS=4>"),
    (8, 1000, 1024, 128, torch.float16, True, "pipe_grouped_kernel<XR=8,CT=1,KP=2,NS=2>"),
    (12, 4100, 4096, 64, torch.bfloat16, False, "pipe_grouped_kernel<XR=16,CT=1,KP=2,NS=4>"),
    (32, 700, 2048, 32, torch.bfloat16, True, "pipe_grouped_kernel<XR=32,CT=1,KP=2,NS=2>"),
    (17, 64, 1024, 128, torch.float16, True, "pipe_grouped_kernel<XR=32,CT=1,KP=2,NS=2>"),
    (4, 500, 768, 32, torch.bfloat16, True, "grouped_generic_kernel"),   # k the ring cannot tile
]


@pytest.mark.parametrize("m,n,k,g,dtype,bias,kernel", SKINNY)
def test_grouped_skinny(m, n, k, g, dtype, bias, kernel):
    print(f"grouped skinny m={m} n={n} k={k} g={g} {kernel}", flush=True)
    w, x, b = _case(m * 31 + n + k, m, n, k, g, dtype, bias)
    _run_and_check(w, x, b, g, fw.PATH_AUTO, kernel)


GENERIC = [
    # (m, n, k, g, dtype, bias, x_offset)
    (33, 100, 544, 32, torch.bfloat16, True, 0),    # k % 256 != 0 above 32 tokens
    (70, 45, 320, 64, torch.float16, False, 0),     # k % 256 != 0, ragged m and n
    (1, 77, 8320, 128, torch.bfloat16, True, 0),
    (5, 130, 1024, 32, torch.float16, True, 1),     # x not 16-byte aligned
    (3, 20, 0, 32, torch.bfloat16, True, 0),        # k = 0: y = bias
]


@pytest.mark.parametrize("m,n,k,g,dtype,bias,xoff", GENERIC)
def test_grouped_generic(m, n, k, g, dtype, bias, xoff):
    print(f"grouped generic m={m} n={n} k={k} g={g}", flush=True)
    if k == 0:
        b = torch.randn(n, device=DEV).to(dtype)
        y = nan_like((m, n), dtype, DEV)
        st = fw.fp8w_linear_grouped(0, fw.BF16, m, 0, 0, 0, g, b.data_ptr(), n, y.data_ptr(), 0)
        torch.cuda.synchronize()
        assert st == 0
        assert torch.equal(y, b[None, :].expand(m, n))
        return
    w, x, b = _case(m + n + k, m, n, k, g, dtype, bias)
    _run_and_check(w, x, b, g, fw.PATH_AUTO, "grouped_generic_kernel", x_offset=xoff)


BATCH = [
    # (m, n, k, g, dtype, bias, kernel): the batch GEMM with group scales, every
    # tile it plans for each group size, ragged channel and token tails, the
    # shortest ring (k = 256) and k stagger over the XCDs
    (33, 100, 512, 32, torch.bfloat16, True, "batch_grouped_kernel<BN=64,BM=32,W=2>"),
    (40, 300, 1024, 128, torch.float16, False, "batch_grouped_kernel<BN=64,BM=32,W=2>x2+splitk_reduce_kernel"),
    (33, 4100, 768, 64, torch.bfloat16, True, "batch_grouped_kernel<BN=64,BM=32,W=2>"),
    (96, 2000, 2048, 128, torch.bfloat16, True, "batch_grouped_kernel<BN=64,BM=32,W=2>x2+splitk_reduce_kernel"),
    (100, 9000, 2048, 32, torch.float16, True, "batch_grouped_kernel<BN=64,BM=64,W=4>"),
    (200, 10000, 512, 64, torch.bfloat16, False, "batch_grouped_kernel<BN=64,BM=64,W=4>"),
    (300, 4096, 4096, 64, torch.float16, True, "batch_grouped_kernel<BN=128,BM=64,W=8>"),
    (1000, 3000, 256, 128, torch.bfloat16, True, "batch_grouped_kernel<BN=128,BM=64,W=8>"),
    # k split over workgroups (fp32 partial sums that hold the group scales)
    (33, 1000, 3072, 32, torch.float16, True, "batch_grouped_kernel<BN=64,BM=32,W=2>x6+splitk_reduce_kernel"),
    (90, 1000, 1536, 128, torch.bfloat16, False, "batch_grouped_kernel<BN=64,BM=32,W=2>x3+splitk_reduce_kernel"),
    (150, 1200, 4096, 64, torch.bfloat16, True, "batch_grouped_kernel<BN=64,BM=64,W=4>x4+splitk_reduce_kernel"),
    (128, 4096, 4096, 128, torch.float16, True, "batch_grouped_kernel<BN=128,BM=64,W=8>x4+splitk_reduce_kernel"),
    # fewer channels than one tile (rows past n read the last row, never stored)
    (33, 1, 256, 32, torch.bfloat16, True, "batch_grouped_kernel<BN=64,BM=32,W=2>"),
    (257, 63, 512, 64, torch.float16, True, "batch_grouped_kernel<BN=64,BM=32,W=2>"),
    (33, 5, 1024, 128, torch.bfloat16, False, "batch_grouped_kernel<BN=64,BM=32,W=2>x2+splitk_reduce_kernel"),
]


@pytest.mark.parametrize("m,n,k,g,dtype,bias,kernel", BATCH)
def test_grouped_batch(m, n, k, g, dtype, bias, kernel):
    print(f"grouped batch m={m} n={n} k={k} g={g} {kernel}", flush=True)
    w, x, b = _case(m * 7 + n + k + g, m, n, k, g, dtype, bias)
    y = _run_and_check(w, x, b, g, fw.PATH_AUTO, kernel)  # allocates the workspace a split plan asks for
    if "splitk" in kernel:
        # no workspace: the single-pass plan, within the gate and within fp32
        # summation-order rounding of the split result
        y1 = _run_and_check(w, x, b, g, fw.PATH_AUTO, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
        assert np.allclose(y1.double().cpu().numpy(), y.double().cpu().numpy(), rtol=2e-2, atol=1e-2)


@pytest.mark.parametrize("m,k,g", [(1, 1024, 32), (4, 2048, 64), (24, 1024, 128), (32, 1024, 32),
                                   (40, 1024, 64), (65, 2048, 32)])
def test_grouped_paths_agree(m, k, g):
    """Forced paths on the same covered shape each pass the gate and agree
    within fp32 summation-order rounding."""
    n = 300
    w, x, b = _case(m + k + g, m, n, k, g, torch.bfloat16, True)
    paths = [fw.PATH_FALLBACK] + ([fw.PATH_SKINNY] if m <= 32 else []) + ([fw.PATH_GEMV] if m == 1 else []) + \
        [fw.PATH_BATCH]
    outs = [_run_and_check(w, x, b, g, p).double().cpu().numpy() for p in paths]
    for o in outs[1:]:
        assert np.allclose(o, outs[0], rtol=2e-2, atol=1e-2)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_dequantize_grouped_bits(dtype):
    n, k, g = 50, 640, 64
    w = _weights(3, n, k, g)
    q, s = fw.quantize_grouped(torch.from_numpy(w).to(DEV), g)
    out = fw.dequantize_grouped(q, s, dtype).cpu()
    qn, sn = q.cpu().numpy(), s.cpu().numpy()
    # fl32(value * scale): every e4m3 value is exact in fp32, so numpy's IEEE
    # float32 product is the reference; then the dtype's round to nearest even
    prod = (oracle.decode(qn).astype(np.float32) * np.repeat(sn, g, axis=1)).astype(np.float32)
    if dtype == torch.float32:
        assert_same_bits(out.numpy(), prod, "fp32 dequantize")
    else:
        ref = torch.from_numpy(prod).to(dtype)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("shape,m,g", [((14336, 4096), 1, 128), ((4096, 14336), 1, 32),
                                       ((14336, 4096), 16, 32), ((14336, 4096), 32, 128),
                                       ((4096, 4096), 16, 64), ((14336, 4096), 128, 128),
                                       ((4096, 14336), 64, 32)])
def test_grouped_full_size(shape, m, g):
    """Decode- and sweep-sized layers: every output of the call against the oracle."""
    n, k = shape
    print(f"grouped full size {shape} m={m} g={g}", flush=True)
    w = workloads.weight_normal(7, n // 1024 + k // 1024, n, k, 0.02)
    x = workloads.activations(7, m, m, k, torch.bfloat16)
    _run_and_check(w, x, None, g, fw.PATH_AUTO)


def test_grouped_batch_zero_token_rows_give_bias():
    """Token rows of zeros through the grouped batch GEMM give the bias exactly,
    single pass and split."""
    for (m, n, k, g) in [(70, 500, 512, 32), (40, 300, 2048, 128)]:
        w, x, b = _case(m + n + k, m, n, k, g, torch.float16, True)
        x[[0, 33, m - 1]] = 0.0
        q, s = fw.quantize_grouped(torch.from_numpy(w).to(DEV), g)
        xd = x.to(DEV)
        assert fw.fp8w_linear_grouped_path(m, n, k, g, fw.FP16, xd.data_ptr(), q.data_ptr()) == fw.PATH_BATCH
        y = fw.linear_grouped(xd, q, s, b.to(DEV))
        torch.cuda.synchronize()
        for r in (0, 33, m - 1):
            assert torch.equal(y[r].cpu(), b)
