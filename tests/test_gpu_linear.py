"""GPU parity of the linear layer (fp8w_linear and its three paths) and of the
exported dequantize, at sizes the oracle finishes in seconds that still span
several tiles and ragged tails.

Sources: "FP8 weight-only (precision: fp8_weights)", sections "The contract"
and "Dequantise in registers"; "Inference with NVFP4/MXFP8" (cuTile-rs), the
all-ones check; "Skill: Write an FP8 Kernel", step 7 (scale = 0).
"""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_gate, assert_same_bits, nan_like, oracle_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
PATHS = {fw.PATH_GEMV: "gemv", fw.PATH_SKINNY: "skinny", fw.PATH_FALLBACK: "fallback", fw.PATH_BATCH: "batch"}


def _prepare(case):
    w = torch.from_numpy(case.layer.w).to(DEV)
    q, s = fw.quantize(w)
    x = case.x.to(DEV)
    b = None if case.layer.bias is None else case.layer.bias.to(DEV)
    return q, s, x, b


def _check(case, path=fw.PATH_AUTO, expect_path=None):
    q, s, x, b = _prepare(case)
    m, k = case.x.shape
    n = case.layer.w.shape[0]
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    assert_same_bits(q.cpu().numpy(), q_ref, "codes")
    if expect_path is not None:
        assert fw.linear_path(x, q) == expect_path
    y = nan_like((m, n), case.x.dtype, DEV)
    fw.linear(x, q, s, b, out=y, path=path)
    torch.cuda.synchronize()
    assert_gate(y.double().cpu().numpy(), y_ref, x64, amax, f"{case.layer.name} m={m} path={path}")
    return y


SMALL = [
    # (m, n, k, dtype, bias, expected auto path)
    (1, 1024, 1024, torch.bfloat16, True, fw.PATH_GEMV),
    (1, 17, 256, torch.bfloat16, True, fw.PATH_GEMV),
    (1, 300, 4352, torch.float16, False, fw.PATH_GEMV),
    (1, 64, 14336, torch.bfloat16, True, fw.PATH_GEMV),
    (2, 272, 512, torch.float16, True, fw.PATH_SKINNY),
    (4, 100, 768, torch.bfloat16, False, fw.PATH_SKINNY),
    (8, 33, 4096, torch.bfloat16, True, fw.PATH_SKINNY),
    (16, 512, 1024, torch.float16, True, fw.PATH_SKINNY),
    (17, 48, 2048, torch.bfloat16, True, fw.PATH_SKINNY),
    (22, 130, 1280, torch.float16, True, fw.PATH_SKINNY),
    (32, 256, 4096, torch.bfloat16, False, fw.PATH_SKINNY),
    (6, 8200, 256, torch.bfloat16, True, fw.PATH_SKINNY),
    (12, 40, 768, torch.float16, False, fw.PATH_SKINNY),
    (20, 8192, 512, torch.float16, True, fw.PATH_SKINNY),
    (3, 8192, 1024, torch.bfloat16, True, fw.PATH_SKINNY),
    (33, 64, 512, torch.bfloat16, True, fw.PATH_BATCH),
    (300, 200, 768, torch.float16, False, fw.PATH_BATCH),
    (70, 40, 300, torch.float16, True, fw.PATH_FALLBACK),
    (1, 77, 8200, torch.bfloat16, True, fw.PATH_GEMV),         # 8-code GEMV: k % 256 != 0
    (3, 50, 1, torch.bfloat16, True, fw.PATH_FALLBACK),
    (5, 31, 37, torch.float16, False, fw.PATH_FALLBACK),
    (4, 128, 200, torch.bfloat16, True, fw.PATH_FALLBACK),
    (40, 300, 1000, torch.float16, True, fw.PATH_FALLBACK),    # 2 token tiles, 488-value k tail
    (7, 16500, 776, torch.bfloat16, False, fw.PATH_SKINNY),    # unaligned-code path, wide layer, 264-value tail
    (7, 16500, 504, torch.bfloat16, False, fw.PATH_FALLBACK),  # k < 512: the fallback's ring, 248-value tail
    (12, 70, 264, torch.bfloat16, True, fw.PATH_FALLBACK),     # shortest ring (2 stages), 8-value tail
]


@pytest.mark.parametrize("m,n,k,dtype,bias,path", SMALL)
def test_linear_small_parity(m, n, k, dtype, bias, path):
    print(f"linear m={m} n={n} k={k} {dtype} bias={bias} path={PATHS[path]}", flush=True)
    case = workloads.random_case(m * 1000 + n, m, n, k, dtype, with_bias=bias)
    _check(case, expect_path=path)


PIPE = [
    # (m, n, k, dtype, kernel the dispatcher must pick): every ring shape and
    # activation-row count of the direct-to-LDS kernel, ragged channel tails
    (2, 12300, 1024, torch.bfloat16, "pipe_kernel<XR=4,CT=4,KP=1,NS=4>"),
    (5, 8200, 1024, torch.float16, "pipe_kernel<XR=8,CT=2,KP=1,NS=4>"),
    (7, 8250, 512, torch.bfloat16, "pipe_kernel<XR=8,CT=2,KP=1,NS=2>"),
    (9, 200, 2048, torch.bfloat16, "pipe_kernel<XR=12,CT=1,KP=2,NS=4>"),
    (16, 4100, 1024, torch.float16, "pipe_kernel<XR=16,CT=1,KP=2,NS=2>"),
    (19, 16400, 512, torch.bfloat16, "pipe_kernel<XR=24,CT=4,KP=1,NS=2>"),
    (24, 12288, 2048, torch.float16, "pipe_kernel<XR=24,CT=3,KP=1,NS=4>"),
    (3, 12288, 512, torch.bfloat16, "pipe_kernel<XR=4,CT=3,KP=1,NS=2>"),
    (16, 12288, 4096, torch.bfloat16, "pipe_kernel<XR=16,CT=3,KP=1,NS=4>"),
    (32, 8192, 3072, torch.float16, "pipe_kernel<XR=32,CT=2,KP=1,NS=4>"),
    (32, 300, 4096, torch.bfloat16, "pipe_kernel<XR=32,CT=1,KP=2,NS=4>"),
    (3, 16500, 1536, torch.bfloat16, "pipe_kernel<XR=4,CT=4,KP=1,NS=2>"),
    (6, 8192, 2048, torch.bfloat16, "pipe_kernel<XR=8,CT=2,KP=2,NS=4>"),
    (12, 9000, 4096, torch.float16, "pipe_kernel<XR=12,CT=2,KP=2,NS=4>"),
    (10, 8300, 1024, torch.bfloat16, "pipe_kernel<XR=12,CT=2,KP=1,NS=4>"),
    (13, 4100, 2048, torch.float16, "pipe_kernel<XR=16,CT=1,KP=2,NS=4>"),
    (11, 12288, 1024, torch.bfloat16, "pipe_kernel<XR=12,CT=3,KP=1,NS=4>"),
    (12, 14400, 1024, torch.float16, "pipe_kernel<XR=12,CT=4,KP=1,NS=4>"),
    (20, 8200, 2048, torch.bfloat16, "pipe_kernel<XR=24,CT=4,KP=1,NS=4>x2+splitk_reduce_kernel"),
    (32, 8192, 4096, torch.float16, "pipe_kernel<XR=32,CT=4,KP=1,NS=4>x2+splitk_reduce_kernel"),
    (17, 4100, 10240, torch.float16, "pipe_kernel<XR=24,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"),
    (28, 4100, 2048, torch.bfloat16, "pipe_kernel<XR=32,CT=4,KP=1,NS=2>x4+splitk_reduce_kernel"),
    (16, 4096, 14336, torch.bfloat16, "pipe_kernel<XR=16,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"),
    (12, 4100, 14336, torch.float16, "pipe_kernel<XR=12,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"),
    (24, 5000, 12288, torch.bfloat16, "pipe_kernel<XR=24,CT=4,KP=1,NS=4>x4+splitk_reduce_kernel"),
    (32, 4096, 6144, torch.bfloat16, "pipe_kernel<XR=32,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"),
    # eight tiles on three-stage rings, stage counts 32, 33 and 34 (every
    # remainder mod 3), ragged channel tail
    (13, 16400, 8192, torch.float16, "pipe_kernel<XR=16,CT=8,KP=1,NS=3>"),
    (22, 16400, 8448, torch.bfloat16, "pipe_kernel<XR=24,CT=8,KP=1,NS=3>"),
    (32, 16400, 8704, torch.float16, "pipe_kernel<XR=32,CT=8,KP=1,NS=3>"),
    # an odd number of 256-column stages: splits of whole stages, uneven by at
    # most one (43 stages in four, 29 in three, 22 in four), three-stage rings,
    # four- and two-tile workgroups, ragged channel counts, one split plan
    # below 9 tokens
    (12, 4096, 11008, torch.bfloat16, "pipe_kernel<XR=12,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"),
    (32, 5120, 13824, torch.float16, "pipe_kernel<XR=32,CT=4,KP=1,NS=3>x3+splitk_reduce_kernel"),
    (3, 4100, 13824, torch.bfloat16, "pipe_kernel<XR=4,CT=4,KP=1,NS=3>x3+splitk_reduce_kernel"),
    (20, 2048, 5632, torch.float16, "pipe_kernel<XR=24,CT=2,KP=1,NS=3>x4+splitk_reduce_kernel"),
    (9, 2100, 7424, torch.bfloat16, "pipe_kernel<XR=12,CT=2,KP=1,NS=3>x3+splitk_reduce_kernel"),
    (17, 4096, 7168, torch.float16, "pipe_kernel<XR=24,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"),
    # k split from 12 tokens on long rows of 8192-channel layers
    (12, 8200, 20480, torch.bfloat16, "pipe_kernel<XR=12,CT=4,KP=1,NS=4>x2+splitk_reduce_kernel"),
]


@pytest.mark.parametrize("m,n,k,dtype,kernel", PIPE)
def test_pipe_kernel_parity(m, n, k, dtype, kernel):
    print(f"pipe m={m} n={n} k={k} {dtype} {kernel}", flush=True)
    assert fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, fw.BF16 if dtype == torch.bfloat16 else fw.FP16,
                                 0, 0) == kernel
    case = workloads.random_case(31 * m + n + k, m, n, k, dtype, with_bias=(m % 2 == 1))
    _check(case, expect_path=fw.PATH_SKINNY)


RING4 = [
    # (m, n, k, dtype, bias, byte offset of q, kernel the dispatcher must pick):
    # codes the 16-byte kernels cannot load. CB=8: rows 8-byte aligned that
    # are 16-byte aligned or alternate (k % 16 == 8), 16-byte loads from each
    # workgroup's first 16-byte boundary, workgroups of one row parity; CB=4:
    # 4-byte loads (q 4 bytes off, or every row 8 bytes off). Every ring shape
    # either uses, columns outside the ring of 8 to 504, ragged channels.
    (1, 77, 8200, torch.bfloat16, True, 4, "pipe_kernel<XR=4,CT=1,KP=2,NS=4,CB=4>"),
    (4, 4096, 14344, torch.float16, True, 0, "pipe_kernel<XR=4,CT=1,KP=2,NS=4,CB=8>"),
    (2, 16500, 1032, torch.bfloat16, False, 0, "pipe_kernel<XR=4,CT=4,KP=1,NS=2,CB=8>"),
    (4, 12300, 4344, torch.float16, True, 0, "pipe_kernel<XR=4,CT=4,KP=1,NS=4,CB=8>"),
    (6, 12288, 2056, torch.bfloat16, True, 0, "pipe_kernel<XR=8,CT=2,KP=1,NS=4,CB=8>"),
    (8, 8200, 2056, torch.float16, False, 0, "pipe_kernel<XR=8,CT=2,KP=2,NS=4,CB=8>"),
    (16, 9000, 1288, torch.bfloat16, True, 0, "pipe_kernel<XR=16,CT=2,KP=1,NS=4,CB=8>"),
    (17, 8300, 1544, torch.float16, True, 0, "pipe_kernel<XR=32,CT=2,KP=1,NS=2,CB=8>"),
    (9, 300, 776, torch.bfloat16, False, 0, "pipe_kernel<XR=16,CT=2,KP=1,NS=2,CB=8>"),
    (12, 1000, 4104, torch.float16, True, 0, "pipe_kernel<XR=16,CT=1,KP=2,NS=4,CB=8>"),
    (32, 300, 2056, torch.bfloat16, True, 0, "pipe_kernel<XR=32,CT=1,KP=2,NS=2,CB=8>"),
    (24, 5000, 1528, torch.bfloat16, False, 0, "pipe_kernel<XR=32,CT=1,KP=2,NS=2,CB=8>"),
    (5, 28672, 1032, torch.bfloat16, True, 0, "pipe_kernel<XR=8,CT=4,KP=1,NS=2,CB=8>"),
    (16, 4096, 4096, torch.bfloat16, True, 4, "pipe_kernel<XR=16,CT=1,KP=2,NS=4,CB=4>"),
    (3, 14336, 4096, torch.float16, True, 8, "pipe_kernel<XR=4,CT=4,KP=1,NS=4,CB=4>"),
    (32, 14336, 4096, torch.bfloat16, False, 12, "pipe_kernel<XR=32,CT=4,KP=1,NS=4,CB=4>"),
    (3, 100, 520, torch.float16, True, 8, "pipe_kernel<XR=4,CT=2,KP=1,NS=2,CB=8>"),     # row 0 the shifted one
    (7, 33, 1032, torch.bfloat16, True, 8, "pipe_kernel<XR=8,CT=1,KP=2,NS=2,CB=8>"),    # odd n: last odd workgroup idle
    (13, 65, 2312, torch.float16, False, 8, "pipe_kernel<XR=16,CT=1,KP=2,NS=4,CB=8>"),
    (10, 333, 4480, torch.bfloat16, True, 0, "pipe_kernel<XR=16,CT=1,KP=2,NS=4,CB=8>"),  # aligned rows, 384 left over
    (20, 4100, 4112, torch.float16, True, 0, "pipe_kernel<XR=32,CT=1,KP=2,NS=2,CB=8>"),
    (32, 129, 8200, torch.bfloat16, True, 8, "pipe_kernel<XR=32,CT=1,KP=2,NS=2,CB=8>"),
    (22, 70, 8200, torch.float16, False, 0, "pipe_kernel<XR=32,CT=1,KP=2,NS=2,CB=8>"),
    (2, 8200, 2056, torch.bfloat16, True, 0, "pipe_kernel<XR=4,CT=2,KP=2,NS=4,CB=8>"),
]


@pytest.mark.parametrize("m,n,k,dtype,bias,qoff,kernel", RING4)
def test_ring4_parity(m, n, k, dtype, bias, qoff, kernel):
    """Codes whose rows are only 4-byte aligned: every output against the oracle."""
    print(f"ring4 m={m} n={n} k={k} {dtype} bias={bias} qoff={qoff} {kernel}", flush=True)
    case = workloads.random_case(17 * m + n + k, m, n, k, dtype, with_bias=bias)
    q0, s, x, b = _prepare(case)
    qbuf = torch.zeros(n * k + 16, dtype=torch.uint8, device=DEV)
    q = qbuf[qoff:qoff + n * k].view(n, k)
    q.copy_(q0)
    act = fw.BF16 if dtype == torch.bfloat16 else fw.FP16
    assert fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, act, x.data_ptr(), q.data_ptr()) == kernel
    assert fw.linear_path(x, q) == fw.PATH_SKINNY
    assert fw.workspace_bytes(x, q) == 0
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    assert_same_bits(q.cpu().numpy(), q_ref, "codes")
    y = nan_like((m, n), dtype, DEV)
    fw.linear(x, q, s, b, out=y)
    torch.cuda.synchronize()
    assert_gate(y.double().cpu().numpy(), y_ref, x64, amax, f"ring4 m={m} n={n} k={k} qoff={qoff}")


GEMV8 = [
    # (m, n, k, dtype, bias, byte offset of q, kernel): one token on codes whose
    # rows are only 8-byte aligned, every GEMV instance, pass tails
    (1, 77, 8200, torch.bfloat16, True, 0, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),   # k % 16 == 8: rows alternate
    (1, 77, 8200, torch.bfloat16, True, 8, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),   # row 0 the shifted one
    (1, 4096, 4104, torch.float16, False, 0, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),
    (1, 300, 264, torch.bfloat16, True, 0, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),   # 16 chunks: one partial group
    (1, 1, 1032, torch.float16, True, 8, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),     # one row: odd workgroup idle
    (1, 5, 4360, torch.bfloat16, False, 0, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),   # odd n: a row pair short
    (1, 12300, 8200, torch.float16, True, 0, "gemv_shift_kernel<R=4,U=2,NT=128>"),
    (1, 12301, 8200, torch.bfloat16, False, 8, "gemv_shift_kernel<R=4,U=2,NT=128>"),
    (1, 4096, 4096, torch.bfloat16, True, 8, "gemv_kernel<R=2,U=2,NT=64,DB,CH=8>"),  # every row 8 bytes off
    (1, 300, 280, torch.float16, True, 8, "gemv_shift_kernel<R=2,U=2,NT=64,DB>"),
    (1, 12300, 8192, torch.float16, True, 8, "gemv_kernel<R=4,U=2,NT=128,CH=8>"),
    (1, 1000, 4112, torch.bfloat16, True, 0, "gemv_kernel<R=2,U=2,NT=64,DB>"),  # k % 16 == 0: 16-code chunks, pass tail
    (1, 4100, 6656, torch.float16, True, 0, "gemv_kernel<R=2,U=1,NT=64,DB>"),   # one-pass groups, odd group count, pass tail
    (1, 5000, 14336, torch.bfloat16, False, 0, "gemv_kernel<R=2,U=1,NT=64,DB>"),  # fourteen one-pass groups
]


@pytest.mark.parametrize("m,n,k,dtype,bias,qoff,kernel", GEMV8)
def test_gemv8_parity(m, n, k, dtype, bias, qoff, kernel):
    """One token, codes whose rows are only 8-byte aligned: every output against the oracle."""
    print(f"gemv8 n={n} k={k} {dtype} bias={bias} qoff={qoff} {kernel}", flush=True)
    case = workloads.random_case(23 * n + k, m, n, k, dtype, with_bias=bias)
    q0, s, x, b = _prepare(case)
    qbuf = torch.zeros(n * k + 16, dtype=torch.uint8, device=DEV)
    q = qbuf[qoff:qoff + n * k].view(n, k)
    q.copy_(q0)
    act = fw.BF16 if dtype == torch.bfloat16 else fw.FP16
    assert fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, act, x.data_ptr(), q.data_ptr()) == kernel
    assert fw.linear_path(x, q) == fw.PATH_GEMV
    assert fw.workspace_bytes(x, q) == 0
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    y = nan_like((m, n), dtype, DEV)
    fw.linear(x, q, s, b, out=y)
    torch.cuda.synchronize()
    assert_gate(y.double().cpu().numpy(), y_ref, x64, amax, f"gemv8 n={n} k={k} qoff={qoff}")


NARROW = [
    # (m, n, k, dtype, kernel the dispatcher must pick): every instance of the
    # narrow-layer kernel, ragged channel tails, rings that run their main loop
    # (more stages than the ring holds) and rings that do not, every token tile
    (2, 4096, 4096, torch.bfloat16, "narrow_kernel<MT=1,W=4,NS=4>"),
    (5, 1000, 4096, torch.float16, "narrow_kernel<MT=1,W=4,NS=4>"),
    (9, 4100, 8192, torch.bfloat16, "narrow_kernel<MT=1,W=4,NS=4>"),
    (16, 33, 4096, torch.float16, "narrow_kernel<MT=1,W=8,NS=2,QL>"),
    (16, 4096, 4096, torch.bfloat16, "narrow_kernel<MT=1,W=8,NS=2,QL>"),
    (10, 4100, 4096, torch.float16, "narrow_kernel<MT=1,W=8,NS=2,QL>"),
    (11, 2000, 4096, torch.float16, "narrow_kernel<MT=1,W=8,NS=2,QL>"),
    (13, 1000, 8192, torch.bfloat16, "narrow_kernel<MT=1,W=8,NS=2,QL>"),
    (12, 4096, 7168, torch.bfloat16, "narrow_kernel<MT=1,W=7,NS=2,QL>"),
    (11, 4096, 14336, torch.bfloat16, "narrow_kernel<MT=1,W=7,NS=2,QL>"),
    (6, 500, 14336, torch.float16, "narrow_kernel<MT=1,W=7,NS=2,QL>"),
    (15, 4100, 21504, torch.float16, "narrow_kernel<MT=1,W=7,NS=2,QL>"),
    (5, 500, 7168, torch.float16, "narrow_kernel<MT=1,W=7,NS=4>"),
    (3, 500, 14336, torch.float16, "narrow_kernel<MT=1,W=7,NS=4>"),
    (17, 4096, 2048, torch.bfloat16, "narrow_kernel<MT=2,W=4,NS=2>"),
    (24, 300, 8192, torch.float16, "narrow_kernel<MT=2,W=4,NS=2>"),
    (20, 4100, 6144, torch.bfloat16, "narrow_kernel<MT=2,W=4,NS=2>"),
]


@pytest.mark.parametrize("m,n,k,dtype,kernel", NARROW)
def test_narrow_kernel_parity(m, n, k, dtype, kernel):
    print(f"narrow m={m} n={n} k={k} {dtype} {kernel}", flush=True)
    assert fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, fw.BF16 if dtype == torch.bfloat16 else fw.FP16,
                                 0, 0) == kernel
    case = workloads.random_case(17 * m + n + k, m, n, k, dtype, with_bias=(m % 2 == 0))
    _check(case, expect_path=fw.PATH_SKINNY)


def _ql_draw(i):
    r = np.random.default_rng([5574, i])
    if r.random() < 0.5:
        k = 4096 * int(r.integers(1, 4))
        m = int(r.integers(10, 17))
    else:
        k = 7168 * int(r.integers(1, 4))
        m = int(r.integers(6, 17))
    n = int(r.integers(1, 8192))
    n = max(1, min(n, int(3e7) // k))
    dtype = torch.bfloat16 if r.random() < 0.5 else torch.float16
    return (i, m, n, k, dtype, bool(r.random() < 0.6))


@pytest.mark.parametrize("case", [_ql_draw(i) for i in range(24)],
                         ids=lambda c: f"{c[0]}-m{c[1]}-n{c[2]}-k{c[3]}")
def test_narrow_ql_random_shapes(case):
    """Seeded shapes that take the QL narrow kernels (each token's activation
    parts loaded by neighbouring lanes, moved by ds_bpermute): every token count
    they take, ragged channel counts, one to three 4096- or 7168-column ring
    lengths, both activation types, with and without bias."""
    i, m, n, k, dtype, bias = case
    act = fw.BF16 if dtype == torch.bfloat16 else fw.FP16
    name = fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, act, 0, 0)
    print(f"ql sweep {i} m={m} n={n} k={k} {dtype} {name}", flush=True)
    assert name.startswith("narrow_kernel<") and name.endswith(",QL>")
    case = workloads.random_case(7300 + i, m, n, k, dtype, with_bias=bias)
    _check(case, expect_path=fw.PATH_SKINNY)


@pytest.mark.parametrize("m,n,k,splits", [(24, 8256, 4096, 2), (20, 4160, 10240, 4)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_split_k_matches_single_pass(m, n, k, splits, dtype):
    """A shape that splits k when given workspace: with it (workgroup rows of
    fp32 partial sums, then the reduce kernel) and without it (single pass) both
    pass the gate, and agree to fp32 summation-order rounding."""
    act = fw.BF16 if dtype == torch.bfloat16 else fw.FP16
    need = splits * m * n * 4
    assert fw.fp8w_linear_workspace_bytes(m, n, k, act, 0, 0, 0) == need
    case = workloads.random_case(4242, m, n, k, dtype, with_bias=True)
    q, s, x, b = _prepare(case)
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    outs = []
    for ws in (None, torch.empty(0, dtype=torch.uint8, device=DEV)):
        y = nan_like((m, n), dtype, DEV)
        fw.linear(x, q, s, b, out=y, workspace=ws)
        torch.cuda.synchronize()
        yv = y.double().cpu().numpy()
        assert_gate(yv, y_ref, x64, amax, f"split={ws is None}")
        outs.append(yv)
    assert np.allclose(outs[0], outs[1], rtol=2e-2, atol=1e-2)
    # whatever the workspace holds when a call starts, and when calls reuse it
    # without clearing: the same bits
    for fill in (0x7F, 0x00, 0xFF):
        ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        for _ in range(3):
            y2 = nan_like((m, n), dtype, DEV)
            fw.linear(x, q, s, b, out=y2, workspace=ws)
            torch.cuda.synchronize()
            assert np.array_equal(y2.double().cpu().numpy(), outs[0]), f"workspace filled with {fill:#x}"


@pytest.mark.parametrize("m,k", [(1, 256), (1, 4096), (2, 1024), (16, 768), (17, 512), (32, 2048)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_every_path_matches_the_oracle(m, k, dtype):
    """Forced paths on covered shapes: the GEMV (m == 1), the skinny MFMA kernel,
    the batch GEMM and the fallback each pass the gate on the same inputs."""
    n = 200
    case = workloads.random_case(7 + m + k, m, n, k, dtype)
    paths = [fw.PATH_SKINNY, fw.PATH_FALLBACK, fw.PATH_BATCH] + ([fw.PATH_GEMV] if m == 1 else [])
    outs = {}
    for p in paths:
        print(f"forced path {PATHS[p]} m={m} k={k} {dtype}", flush=True)
        outs[p] = _check(case, path=p).double().cpu().numpy()
    # the paths differ only in fp32 summation order
    a = outs[fw.PATH_SKINNY]
    for p, o in outs.items():
        assert np.allclose(o, a, rtol=2e-2, atol=1e-2), PATHS[p]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("path,m,n,k", [(fw.PATH_GEMV, 1, 256, 512), (fw.PATH_SKINNY, 2, 256, 512),
                                        (fw.PATH_SKINNY, 6, 256, 512), (fw.PATH_SKINNY, 12, 256, 512),
                                        (fw.PATH_SKINNY, 20, 256, 512), (fw.PATH_FALLBACK, 2, 256, 512),
                                        (fw.PATH_SKINNY, 2, 12288, 1024), (fw.PATH_SKINNY, 12, 256, 2048),
                                        (fw.PATH_SKINNY, 20, 8192, 1024), (fw.PATH_SKINNY, 32, 16384, 512),
                                        (fw.PATH_BATCH, 2, 256, 512), (fw.PATH_BATCH, 40, 300, 256),
                                        (fw.PATH_BATCH, 130, 7168, 256), (fw.PATH_BATCH, 300, 14336, 256)])
def test_all_256_codes_decode_exactly_on_each_path(dtype, path, m, n, k):
    """q[n, :] = n mod 256 for every code, unit scales and a one-hot x: y[n] is
    the exact value of its code (0x7F / 0xFF give NaN). Pins each kernel's
    hardware conversion (fp32 for the GEMV, bf16/f16 for the MFMA operands)
    and its operand layout; the wide shapes take the direct-to-LDS kernel."""
    act = fw.BF16 if dtype == torch.bfloat16 else fw.FP16
    print(f"256 codes {dtype} path={PATHS[path]} m={m} n={n} k={k} "
          f"{fw.fp8w_linear_kernel(path, m, n, k, act, 0, 0)}", flush=True)
    q = (torch.arange(n, dtype=torch.int32) % 256).to(torch.uint8)[:, None].repeat(1, k).contiguous().to(DEV)
    s = torch.ones(n, dtype=torch.float32, device=DEV)
    x = torch.zeros((m, k), dtype=dtype)
    x[0, 5] = 1.0
    if m >= 2:
        x[m - 1, k - 1] = -2.0
    y = nan_like((m, n), dtype, DEV)
    fw.linear(x.to(DEV), q, s, None, out=y, path=path)
    torch.cuda.synchronize()
    yv = y.double().cpu().numpy()
    ref = oracle.decode(np.arange(n) % 256)
    fin = np.isfinite(ref)
    assert np.array_equal(yv[0][fin], ref[fin])
    assert np.all(np.isnan(yv[0][~fin]))
    if m >= 2:
        assert np.array_equal(yv[m - 1][fin], -2.0 * ref[fin])
        for r in range(1, m - 1):  # all-zero activation rows give +-0 (NaN codes give NaN)
            assert np.all(yv[r][fin] == 0.0)


@pytest.mark.parametrize("path", [fw.PATH_GEMV, fw.PATH_SKINNY, fw.PATH_FALLBACK, fw.PATH_BATCH])
def test_all_ones_closed_form(path):
    """x = 1 and rows W[n,:] = c_n: all codes are 0x7E, so y = fl32(c_n/448)*448*K + b."""
    k = 2048
    n = 96
    c = np.linspace(0.001, 2.0, n).astype(np.float32)
    w = np.repeat(c[:, None], k, axis=1)
    m = 1 if path == fw.PATH_GEMV else 3
    b = torch.linspace(-1, 1, n).to(torch.bfloat16)
    q, s = fw.quantize(torch.from_numpy(w).to(DEV))
    assert torch.all(q == 0x7E)
    y = nan_like((m, n), torch.bfloat16, DEV)
    fw.linear(torch.ones((m, k), dtype=torch.bfloat16, device=DEV), q, s, b.to(DEV), out=y, path=path)
    torch.cuda.synchronize()
    expect = (c / np.float32(448.0)).astype(np.float64) * 448.0 * k + b.double().numpy()
    got = y.double().cpu().numpy()
    # fp32 accumulation of 448 * K is exact here; one bf16 rounding of the epilogue remains
    assert np.all(np.abs(got - expect[None, :]) <= np.abs(expect)[None, :] * 2.0 ** -8)


@pytest.mark.parametrize("path", [fw.PATH_GEMV, fw.PATH_SKINNY, fw.PATH_FALLBACK, fw.PATH_BATCH])
def test_zero_rows_give_bias_exactly(path):
    lay = workloads.block_layer(0)
    w = lay.w[:512].copy()
    zero_rows = np.flatnonzero(np.all(w == 0, axis=1))
    w[[5, 77]] = 0.0
    zero_rows = np.union1d(zero_rows, [5, 77])
    m = 1 if path == fw.PATH_GEMV else 5
    case = workloads.Case(workloads.Linear("zero_rows", w, torch.linspace(-3, 3, 512).to(torch.bfloat16)),
                          workloads.activations(41, 0, m, 4096, torch.bfloat16))
    y = _check(case, path=path)
    yz = y[:, zero_rows].cpu()
    assert torch.equal(yz, case.layer.bias[zero_rows][None, :].repeat(m, 1))


@pytest.mark.parametrize("m", [1, 4, 32])
def test_deterministic(m):
    case = workloads.random_case(55, m, 700, 4096, torch.bfloat16)
    q, s, x, b = _prepare(case)
    first = fw.linear(x, q, s, b).clone()
    for _ in range(5):
        again = fw.linear(x, q, s, b)
        assert torch.equal(first.view(torch.int16), again.view(torch.int16))


def test_unaligned_activations_take_the_fallback():
    case = workloads.random_case(61, 4, 96, 1024, torch.bfloat16)
    q, s, _, b = _prepare(case)
    buf = torch.zeros(4 * 1024 + 1, dtype=torch.bfloat16, device=DEV)
    buf[1:] = case.x.reshape(-1).to(DEV)
    x_view = buf[1:].view(4, 1024)
    assert x_view.data_ptr() % 16 != 0
    assert fw.linear_path(x_view, q) == fw.PATH_FALLBACK
    y = nan_like((4, 96), torch.bfloat16, DEV)
    fw.linear(x_view, q, s, b, out=y)
    torch.cuda.synchronize()
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    assert_gate(y.double().cpu().numpy(), y_ref, x64, amax, "unaligned x")


def test_k_zero_gives_bias_and_empty_calls_write_nothing():
    n = 40
    b = torch.linspace(-2, 2, n).to(torch.bfloat16).to(DEV)
    q = torch.empty((n, 0), dtype=torch.uint8, device=DEV)
    s = torch.ones(n, dtype=torch.float32, device=DEV)
    y = nan_like((3, n), torch.bfloat16, DEV)
    fw.linear(torch.empty((3, 0), dtype=torch.bfloat16, device=DEV), q, s, b, out=y)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), b.cpu()[None, :].repeat(3, 1))
    y2 = nan_like((3, n), torch.bfloat16, DEV)
    fw.linear(torch.empty((3, 0), dtype=torch.bfloat16, device=DEV), q, s, None, out=y2)
    torch.cuda.synchronize()
    assert torch.all(y2 == 0)
    # m == 0 and n == 0: nothing to do
    q2 = torch.zeros((n, 256), dtype=torch.uint8, device=DEV)
    out = fw.linear(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), q2, s, b)
    assert out.shape == (0, n)
    q3 = torch.zeros((0, 256), dtype=torch.uint8, device=DEV)
    out = fw.linear(torch.ones((2, 256), dtype=torch.bfloat16, device=DEV), q3,
                    torch.empty(0, dtype=torch.float32, device=DEV))
    assert out.shape == (2, 0)


def test_runs_on_the_callers_stream():
    case = workloads.random_case(71, 8, 333, 2048, torch.float16)
    q, s, x, b = _prepare(case)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        y = fw.linear(x, q, s, b)
    side.synchronize()
    q_ref, s_ref, x64, y_ref, amax = oracle_case(case.layer.w, case.x, case.layer.bias)
    assert_gate(y.double().cpu().numpy(), y_ref, x64, amax, "side stream")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(64, 512), (33, 8200), (7, 13)])
def test_dequantize_matches_oracle(out_dtype, shape):
    """fp8w_dequantize_fallback: fp32 out is exactly q.float() * scale; bf16 / fp16
    round that product to nearest even; without a scale the value is exact."""
    g = np.random.default_rng(shape[1])
    w = (g.standard_normal(shape) * 0.03).astype(np.float32)
    q, s = fw.quantize(torch.from_numpy(w).to(DEV))
    q_np, s_np = q.cpu().numpy(), s.cpu().numpy()
    exact = oracle.dequantize_f64(q_np, s_np)
    f32 = exact.astype(np.float32)  # one rounding of the exact product = the fp32 product
    if out_dtype == torch.float32:
        ref_bits = f32
    elif out_dtype == torch.bfloat16:
        ref_bits = oracle.round_bf16_bits(f32)
    else:
        ref_bits = f32.astype(np.float16)
    got = fw.dequantize(q, s, out_dtype)
    torch.cuda.synchronize()
    got_np = got.cpu().view(torch.int32 if out_dtype == torch.float32 else torch.int16).numpy()
    assert_same_bits(got_np.view(ref_bits.dtype), ref_bits, f"dequantize {out_dtype}")
    unscaled = fw.dequantize(q, None, out_dtype).double().cpu().numpy()
    assert np.array_equal(unscaled, oracle.dequantize_f64(q_np))


def test_stream_read_probe_runs_and_writes_nothing_for_zeros():
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    st = fw.fp8w_stream_read_probe(buf.data_ptr(), buf.numel(), sink.data_ptr(),
                                   torch.cuda.current_stream().cuda_stream)
    assert st == fw.SUCCESS
    torch.cuda.synchronize()
    assert sink.item() == 7
