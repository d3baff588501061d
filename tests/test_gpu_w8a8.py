"""GPU parity of the W8A8 path (per-token activation quantizer and the e4m3 x
e4m3 GEMM) against the oracle.

Source: "Skill: Write an FP8 Kernel", "Required reasoning process" steps 2,
4, 5 and "Correctness requirements". The activation codes and scales must
equal the oracle's bit for bit (the row quantizer on the rows of x); outputs
must pass the gate against the oracle's fp64 W8A8 layer on the same codes,
with the dequantized activations' norm in the gate's second term.
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


def _check(m, n, k, dtype, bias, seed, expect_kernel=None, sampled=False):
    case = workloads.random_case(seed, m, n, k, dtype, with_bias=bias)
    q, s = fw.quantize(torch.from_numpy(case.layer.w).to(DEV))
    x = case.x.to(DEV)
    qx, sx = fw.quantize_activations(x)
    qx_ref, sx_ref, st = oracle.quantize_activations(case.x.float().numpy())
    assert st == 0
    assert_same_bits(sx.cpu().numpy(), sx_ref, "activation scales")
    assert_same_bits(qx.cpu().numpy(), qx_ref, "activation codes")
    if expect_kernel:
        assert fw.fp8w_linear_w8a8_kernel(m, n, k) == expect_kernel
    b = None if case.layer.bias is None else case.layer.bias.to(DEV)
    y = nan_like((m, n), dtype, DEV)
    fw.linear_w8a8(x, q, s, b, out=y)
    torch.cuda.synchronize()
    q_ref, s_ref, _ = oracle.quantize_rows(case.layer.w)
    b64 = None if case.layer.bias is None else case.layer.bias.double().numpy()
    xd = oracle.decode(qx_ref) * sx_ref.astype(np.float64)[:, None]
    amax = oracle.row_amax(case.layer.w)
    yv = y.double().cpu().numpy()
    if not sampled:
        y_ref = oracle.linear_w8a8_f64(qx_ref, sx_ref, q_ref, s_ref, b64)
        assert_gate(yv, y_ref, xd, amax, f"w8a8 m={m} n={n} k={k}")
        return yv
    rows = np.random.default_rng(seed).choice(m, size=min(m, 48), replace=False)
    y_ref = oracle.linear_w8a8_f64(qx_ref[rows], sx_ref[rows], q_ref, s_ref, b64)
    assert_gate(yv[rows], y_ref, xd[rows], amax, f"w8a8 m={m} n={n} k={k} (sampled rows)")
    assert np.all(np.isfinite(yv))
    return yv


CASES = [
    # (m, n, k, dtype, bias)
    (64, 128, 256, torch.bfloat16, True),
    (100, 200, 512, torch.float16, False),      # ragged tiles
    (130, 300, 1024, torch.bfloat16, True),
    (33, 1000, 768, torch.float16, True),
    (1, 64, 256, torch.bfloat16, False),
    (257, 257, 2048, torch.bfloat16, True),
]


@pytest.mark.parametrize("m,n,k,dtype,bias", CASES)
def test_w8a8_small(m, n, k, dtype, bias):
    print(f"w8a8 m={m} n={n} k={k}", flush=True)
    ns = 8 if k % 512 == 0 else 4
    _check(m, n, k, dtype, bias, m + n + k, f"w8a8_kernel<BN=128,BM=64,NS={ns},W=4>")


@pytest.mark.parametrize("m,n,k,dtype,tile", [
    (2048, 4096, 512, torch.bfloat16, "w8a8_kernel<BN=256,BM=128,NS=4,W=8>"),
    (1000, 4000, 768, torch.float16, "w8a8_kernel<BN=128,BM=128,NS=4,W=8>"),     # ragged edges of the 128 x 128 tile
    (700, 4000, 1536, torch.bfloat16, "w8a8_kernel<BN=128,BM=64,NS=4,W=4>"),     # 128 x 64 past 256 workgroups
    (500, 4000, 1536, torch.float16, "w8a8_kernel<BN=128,BM=64,NS=8,W=4>"),      # 128 x 64, 8 stages, ragged
    (2000, 4100, 256, torch.float16, "w8a8_kernel<BN=256,BM=128,NS=4,W=8>"),     # ragged edges of the 256 x 128 tile
])
def test_w8a8_mid_tiles(m, n, k, dtype, tile):
    print(f"w8a8 m={m} n={n} k={k} {tile}", flush=True)
    _check(m, n, k, dtype, True, m + n + k, tile, sampled=True)


def test_w8a8_large_tile():
    print("w8a8 large tile 4096 x 4096 x 1024", flush=True)
    _check(4096, 4096, 1024, torch.bfloat16, True, 5, "w8a8_kernel<BN=256,BM=256,NS=4,W=8>", sampled=True)


def test_w8a8_zero_rows_and_scale_zero():
    """An all-zero token gets scale 0 and codes 0 (no division), so its outputs are the bias."""
    m, n, k = 40, 96, 512
    case = workloads.random_case(9, m, n, k, torch.bfloat16)
    xh = case.x.clone()
    xh[7] = 0
    q, s = fw.quantize(torch.from_numpy(case.layer.w).to(DEV))
    b = case.layer.bias.to(DEV)
    qx, sx = fw.quantize_activations(xh.to(DEV))
    assert sx[7].item() == 0.0
    assert int(qx[7].sum()) == 0
    y = fw.gemm_w8a8(qx, sx, q, s, b)
    torch.cuda.synchronize()
    assert torch.equal(y[7], b)


@pytest.mark.parametrize("i", range(len(workloads.PREFILL_SHAPES)))
def test_w8a8_prefill_workload(i):
    """The prefill workload at full size (M = 2048): activation codes and scales
    bit-exact on every row; outputs against the oracle on every row of the
    [4096, 4096] layer (about 4 s of oracle time on 16 threads) and on 48 seeded
    rows of the two 58.7 MB layers."""
    m = 2048
    lw = workloads.prefill_layer(i)
    n, k = lw.w.shape
    print(f"w8a8 prefill {lw.name} m={m}", flush=True)
    xc = workloads.prefill_x(i, m)
    q, s = fw.quantize(torch.from_numpy(lw.w).to(DEV))
    x = xc.to(DEV)
    qx, sx = fw.quantize_activations(x)
    qx_ref, sx_ref, st = oracle.quantize_activations(xc.float().numpy())
    assert st == 0
    assert_same_bits(sx.cpu().numpy(), sx_ref, "activation scales")
    assert_same_bits(qx.cpu().numpy(), qx_ref, "activation codes")
    assert fw.fp8w_linear_w8a8_kernel(m, n, k) is not None
    y = nan_like((m, n), torch.bfloat16, DEV)
    fw.linear_w8a8(x, q, s, None, out=y)
    torch.cuda.synchronize()
    yv = y.double().cpu().numpy()
    assert np.all(np.isfinite(yv))
    q_ref, s_ref, _ = oracle.quantize_rows(lw.w)
    rows = np.arange(m) if i == 0 else np.random.default_rng(700 + i).choice(m, size=48, replace=False)
    y_ref = oracle.linear_w8a8_f64(qx_ref[rows], sx_ref[rows], q_ref, s_ref, None)
    xd = oracle.decode(qx_ref[rows]) * sx_ref[rows].astype(np.float64)[:, None]
    assert_gate(yv[rows], y_ref, xd, oracle.row_amax(lw.w), f"w8a8 prefill {lw.name} ({rows.size} rows)")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float16])
def test_w8a8_every_code_pair_exact(out_dtype):
    """One-hot codes and unit scales: y[a, b] = value(a) * value(b) from a single
    product, for every pair of finite codes (254 x 254). Each product has at most
    8 significant bits and lies in [2^-18, 448^2], so it is exact in bf16 (and in
    fp16 where it is in range), and the GPU must match it exactly."""
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    m = n = len(codes)
    k = 256
    qx = np.zeros((m, k), dtype=np.uint8)
    qw = np.zeros((n, k), dtype=np.uint8)
    qx[:, 0] = codes
    qw[:, 0] = codes
    ones_m = torch.ones(m, dtype=torch.float32, device=DEV)
    ones_n = torch.ones(n, dtype=torch.float32, device=DEV)
    y = fw.gemm_w8a8(torch.from_numpy(qx).to(DEV), ones_m, torch.from_numpy(qw).to(DEV), ones_n,
                     out_dtype=out_dtype)
    torch.cuda.synchronize()
    v = oracle.decode(codes)
    expect = np.outer(v, v)
    exp_t = torch.from_numpy(expect).to(out_dtype).double().numpy()
    if out_dtype == torch.bfloat16:
        assert np.array_equal(exp_t, expect)  # every product is a bf16 value
    got = y.double().cpu().numpy()
    bad = np.argwhere(got != exp_t)
    assert len(bad) == 0, f"{len(bad)} products differ; first {bad[0]}: got {got[tuple(bad[0])]} want {exp_t[tuple(bad[0])]}"


def test_w8a8_empty_calls_write_nothing_and_results_are_deterministic():
    case = workloads.random_case(31, 300, 520, 512, torch.bfloat16)
    q, s = fw.quantize(torch.from_numpy(case.layer.w).to(DEV))
    x = case.x.to(DEV)
    y = nan_like((300, 520), torch.bfloat16, DEV)
    st = fw.fp8w_linear_w8a8(x.data_ptr(), fw.BF16, 0, 512, q.data_ptr(), s.data_ptr(), 0, 520, y.data_ptr(),
                             0, 0, torch.cuda.current_stream().cuda_stream)
    assert st == fw.SUCCESS
    st = fw.fp8w_gemm_w8a8(0, 0, 300, 512, q.data_ptr(), s.data_ptr(), 0, 0, y.data_ptr(), fw.BF16,
                           torch.cuda.current_stream().cuda_stream)
    assert st == fw.SUCCESS
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()
    y1 = fw.linear_w8a8(x, q, s)
    y2 = fw.linear_w8a8(x, q, s)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
