"""GPU checks of fp8w_linear_noalloc, the entry point for callers that cannot
allocate device memory: through the C ABI it must give the same outputs as
fp8w_linear with a caller-allocated workspace (the same kernels, so bit for
bit), and pass the oracle's gate, on consecutive calls that share the static
scratch, the later ones smaller."""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_gate, nan_like

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _prepare(seed, m, n, k, dtype, bias):
    case = workloads.random_case(seed, m, n, k, dtype, with_bias=bias)
    q, s = fw.quantize(torch.from_numpy(case.layer.w).to(DEV))
    b = None if case.layer.bias is None else case.layer.bias.to(DEV)
    return case, q, s, b


def _reference(case, x, q, s, b):
    """fp8w_linear with the workspace it asks for, allocated by torch."""
    m, k = x.shape
    n = q.shape[0]
    need = fw.workspace_bytes(x, q)
    ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=DEV)
    y = nan_like((m, n), x.dtype, DEV)
    act = fw.BF16 if x.dtype == torch.bfloat16 else fw.FP16
    st = fw.fp8w_linear(x.data_ptr(), act, m, k, q.data_ptr(), s.data_ptr(), 0 if b is None else b.data_ptr(), n,
                        y.data_ptr(), ws.data_ptr() if need else 0, need, torch.cuda.current_stream().cuda_stream)
    assert st == fw.SUCCESS
    return y, need


def _noalloc(x, q, s, b):
    m, k = x.shape
    n = q.shape[0]
    y = nan_like((m, n), x.dtype, DEV)
    act = fw.BF16 if x.dtype == torch.bfloat16 else fw.FP16
    st = fw.fp8w_linear_noalloc(x.data_ptr(), act, m, k, q.data_ptr(), s.data_ptr(),
                                0 if b is None else b.data_ptr(), n, y.data_ptr(),
                                torch.cuda.current_stream().cuda_stream)
    assert st == fw.SUCCESS, fw.fp8w_status_string(st)
    return y


# consecutive calls, each smaller than the one before, on every path that uses
# the scratch: skinny k split in four, then in two, on smaller layers;
# batch k split; the fallback's 16-bit weight (k % 8 != 0); and the GEMV and
# the skinny kernel's unaligned-code path (no scratch); then four-way splits
# of an odd stage count (uneven splits, three-stage rings)
SEQUENCES = [
    [(32, 4096, 14336, torch.bfloat16, False), (20, 4096, 10240, torch.float16, True)],
    [(24, 8192, 4096, torch.bfloat16, True), (17, 8192, 2048, torch.bfloat16, False)],
    [(64, 14336, 4096, torch.bfloat16, False), (40, 2048, 1024, torch.float16, True)],
    [(8, 3000, 1004, torch.bfloat16, True), (3, 700, 524, torch.float16, False)],
    [(1, 4096, 4096, torch.bfloat16, True), (1, 1024, 1024, torch.float16, False)],
    [(16, 2000, 2056, torch.bfloat16, True), (2, 500, 776, torch.float16, False)],
    [(16, 4096, 11008, torch.bfloat16, True), (12, 4096, 7424, torch.float16, False)],
]


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_matches_linear_on_consecutive_calls(seq):
    for i, (m, n, k, dtype, bias) in enumerate(SEQUENCES[seq]):
        case, q, s, b = _prepare(500 + 10 * seq + i, m, n, k, dtype, bias)
        x = case.x.to(DEV)
        path = fw.linear_path(x, q)
        print(f"noalloc seq {seq} call {i}: m={m} n={n} k={k} path={path} "
              f"workspace={fw.workspace_bytes(x, q)}", flush=True)
        y_ref, need = _reference(case, x, q, s, b)
        y = _noalloc(x, q, s, b)
        torch.cuda.synchronize()
        assert need <= fw.SCRATCH_BYTES
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "differs from fp8w_linear"
        q_ref, s_ref, st = oracle.quantize_rows(case.layer.w)
        assert st == 0
        x64 = case.x.double().numpy()
        b64 = None if case.layer.bias is None else case.layer.bias.double().numpy()
        assert_gate(y.double().cpu().numpy(), oracle.linear_f64(x64, q_ref, s_ref, b64), x64,
                    oracle.row_amax(case.layer.w), f"noalloc m={m} n={n} k={k}")


def test_noalloc_refuses_a_fallback_weight_larger_than_the_scratch():
    case, q, s, b = _prepare(590, 4, 4097, 4100, torch.bfloat16, False)  # k % 8 != 0: the fallback
    x = case.x.to(DEV)
    assert fw.linear_path(x, q) == fw.PATH_FALLBACK and fw.workspace_bytes(x, q) > fw.SCRATCH_BYTES
    y = nan_like((4, 4097), torch.bfloat16, DEV)
    st = fw.fp8w_linear_noalloc(x.data_ptr(), fw.BF16, 4, x.shape[1], q.data_ptr(), s.data_ptr(), 0, 4097,
                                y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == fw.ERR_WORKSPACE
    assert torch.isnan(y.float()).all()  # nothing ran
