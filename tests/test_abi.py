"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/fp8w.h declares, and rejects invalid arguments before it
enqueues anything (so no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import fp8_weight_only_amd as fw

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8w.h")

# fake but aligned device addresses: validation must fail before they are used
X = 0x10000000
Q = 0x20000000
S = 0x30000000
B = 0x40000000
Y = 0x50000000
WS = 0x60000000


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"FP8W_API\s+[\w\s\*]+?\b(fp8w_\w+)\s*\(", text)


def test_library_loads_and_exports_every_declared_symbol():
    lib = fw.load()
    names = declared_symbols()
    assert len(names) == 27
    for name in names:
        assert hasattr(lib, name), name
        assert name in fw.EXPORTS, name
    assert fw.fp8w_abi_version() == 1


def test_dynamic_symbol_table_has_only_the_abi():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", fw.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    ours = sorted(l.split()[-1] for l in out.splitlines() if " T " in l and "fp8w" in l)
    assert ours == sorted(declared_symbols())


def test_status_strings():
    for st in range(6):
        s = fw.fp8w_status_string(st)
        assert isinstance(s, str) and s
    assert fw.fp8w_status_string(0) == "success"
    assert "unknown" in fw.fp8w_status_string(99)


def test_path_selection():
    p = fw.fp8w_linear_path
    assert p(1, 4096, 4096, fw.BF16, X, Q, Y) == fw.PATH_GEMV
    assert p(2, 4096, 4096, fw.FP16, X, Q, Y) == fw.PATH_SKINNY
    assert p(32, 4096, 4096, fw.BF16, X, Q, Y) == fw.PATH_SKINNY
    assert p(33, 4096, 4096, fw.BF16, X, Q, Y) == fw.PATH_BATCH
    assert p(4096, 4096, 4096, fw.BF16, X, Q, Y) == fw.PATH_BATCH
    assert p(64, 4096, 4100, fw.BF16, X, Q, Y) == fw.PATH_FALLBACK      # k % 256 != 0
    assert p(64, 4096, 4096, fw.BF16, X, Q + 8, Y) == fw.PATH_FALLBACK  # q not 16-B aligned, m > 32
    assert p(1, 28672, 8200, fw.BF16, X, Q, Y) == fw.PATH_GEMV          # 8-code GEMV: k % 8 == 0, q 8-byte aligned
    assert p(1, 28672, 8200, fw.BF16, X, Q + 4, Y) == fw.PATH_SKINNY    # q 4-byte aligned: 4-byte skinny path
    assert p(1, 4096, 4096, fw.BF16, X, Q + 8, Y) == fw.PATH_GEMV
    assert p(1, 300, 264, fw.BF16, X, Q, Y) == fw.PATH_GEMV             # 8-code GEMV from k = 256
    assert p(2, 300, 264, fw.BF16, X, Q, Y) == fw.PATH_FALLBACK         # 4-byte skinny path from k = 512
    assert p(32, 28672, 8200, fw.BF16, X, Q, Y) == fw.PATH_SKINNY
    assert p(33, 28672, 8200, fw.BF16, X, Q, Y) == fw.PATH_FALLBACK     # unaligned-code path: m <= 32 only
    assert p(4, 100, 520, fw.BF16, X, Q, Y) == fw.PATH_SKINNY
    assert p(4, 100, 504, fw.BF16, X, Q, Y) == fw.PATH_FALLBACK         # unaligned-code path: k >= 512
    assert p(4, 100, 4100, fw.BF16, X, Q, Y) == fw.PATH_FALLBACK        # unaligned-code path: k % 8 == 0
    assert p(4, 100, 4096, fw.BF16, X, Q + 4, Y) == fw.PATH_SKINNY      # q 4-byte aligned
    assert p(4, 100, 4096, fw.BF16, X, Q + 2, Y) == fw.PATH_FALLBACK    # q 2-byte aligned
    assert p(4, 100, 8200, fw.BF16, X + 8, Q, Y) == fw.PATH_FALLBACK    # unaligned-code path: x 16-byte aligned
    assert p(1, 100, 128, fw.BF16, X, Q, Y) == fw.PATH_FALLBACK         # k < 256
    assert p(1, 100, 0, fw.BF16, X, Q, Y) == fw.PATH_FALLBACK           # k == 0
    assert p(1, 4096, 4096, fw.BF16, X + 2, Q, Y) == fw.PATH_FALLBACK   # x not 16-B aligned
    assert p(4, 4096, 4096, fw.BF16, X, Q + 8, Y) == fw.PATH_SKINNY     # q not 16-B aligned: unaligned-code path
    assert p(1, 4096, 4096, fw.BF16, 0, 0, 0) == fw.PATH_GEMV           # NULL = aligned
    assert p(1, 4096, 4096, fw.FP32, X, Q, Y) == -1                     # fp32 activations
    assert p(-1, 4096, 4096, fw.BF16, X, Q, Y) == -1
    assert p(1, -5, 4096, fw.BF16, X, Q, Y) == -1
    assert p(1, 1 << 31, 4096, fw.BF16, X, Q, Y) == -1


def test_kernel_names():
    kn = fw.fp8w_linear_kernel
    A = fw.PATH_AUTO
    assert kn(A, 1, 4096, 4096, fw.BF16, X, Q) == "gemv_kernel<R=2,U=2,NT=64,DB>"
    assert kn(A, 1, 4096, 14336, fw.BF16, X, Q) == "gemv_kernel<R=2,U=1,NT=64,DB>"     # one-pass groups
    assert kn(A, 1, 4096, 11008, fw.BF16, X, Q) == "gemv_kernel<R=2,U=2,NT=64,DB>"     # k % 512 != 0
    assert kn(A, 1, 8192, 8192, fw.BF16, X, Q) == "gemv_kernel<R=2,U=2,NT=64,DB>"
    assert kn(A, 1, 28672, 8192, fw.BF16, X, Q) == "gemv_kernel<R=4,U=2,NT=128>"
    assert kn(A, 16, 14336, 4096, fw.FP16, X, Q) == "pipe_kernel<XR=16,CT=4,KP=1,NS=4>"
    assert kn(A, 32, 28672, 8192, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=8,KP=1,NS=3>"
    assert kn(A, 13, 28672, 8192, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=8,KP=1,NS=3>"
    assert kn(A, 12, 28672, 8192, fw.BF16, X, Q) == "pipe_kernel<XR=12,CT=4,KP=1,NS=2>"
    assert kn(A, 32, 28672, 4096, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=4,KP=1,NS=2>"     # k < 8192
    assert kn(A, 22, 8192, 28672, fw.BF16, X, Q) == "pipe_kernel<XR=24,CT=4,KP=1,NS=4>x2+splitk_reduce_kernel"
    assert kn(A, 8, 8192, 28672, fw.BF16, X, Q) == "pipe_kernel<XR=8,CT=2,KP=2,NS=4>"
    assert kn(A, 12, 8192, 28672, fw.BF16, X, Q) == "pipe_kernel<XR=12,CT=4,KP=1,NS=4>x2+splitk_reduce_kernel"
    assert kn(A, 11, 8192, 28672, fw.BF16, X, Q) == "pipe_kernel<XR=12,CT=2,KP=2,NS=4>"
    assert kn(A, 16, 8192, 14336, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=2,KP=2,NS=4>"      # k < 20480
    assert kn(A, 16, 4096, 11008, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"
    assert kn(A, 8, 4096, 11008, fw.BF16, X, Q) == "seg_kernel<SEG=2,T=2,W=8,U=2,MT=1>"     # splits under 16 stages
    assert kn(A, 4, 5120, 13824, fw.BF16, X, Q) == "pipe_kernel<XR=4,CT=4,KP=1,NS=3>x3+splitk_reduce_kernel"
    assert kn(A, 8, 2048, 5632, fw.BF16, X, Q) == "seg_kernel<SEG=2,T=2,W=8,U=2,MT=1>"
    assert kn(A, 16, 8192, 3072, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=2,KP=1,NS=4>"       # k % 2048 != 0
    assert kn(A, 16, 4096, 4096, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=8,NS=2,QL>"
    assert kn(A, 9, 4096, 4096, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=4,NS=4>"
    assert kn(A, 10, 4096, 4096, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=8,NS=2,QL>"
    assert kn(A, 16, 4100, 2048, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=1,KP=2,NS=4>"     # k % 4096 != 0
    assert kn(A, 16, 4096, 14336, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"
    assert kn(A, 16, 4100, 14336, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"
    assert kn(A, 11, 4096, 14336, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=7,NS=2,QL>"
    assert kn(A, 16, 4096, 28672, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=8,NS=2,QL>"
    assert kn(A, 5, 4096, 14336, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=7,NS=4>"
    assert kn(A, 32, 4096, 14336, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"
    assert kn(A, 28, 4100, 2048, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=4,KP=1,NS=2>x4+splitk_reduce_kernel"  # 2 stages a split
    assert kn(A, 22, 4096, 4096, fw.BF16, X, Q) == "narrow_kernel<MT=2,W=4,NS=2>"
    assert kn(A, 22, 4096, 12288, fw.BF16, X, Q) == "pipe_kernel<XR=24,CT=4,KP=1,NS=4>x4+splitk_reduce_kernel"
    assert kn(A, 17, 6000, 10240, fw.BF16, X, Q) == "pipe_kernel<XR=24,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"
    assert kn(A, 12, 4096, 14336, fw.BF16, X, Q) == "pipe_kernel<XR=12,CT=4,KP=1,NS=3>x4+splitk_reduce_kernel"
    assert kn(A, 6, 4096, 14336, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=7,NS=2,QL>"
    assert kn(A, 25, 4096, 4096, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=4,KP=1,NS=4>x4+splitk_reduce_kernel"
    assert kn(A, 32, 2048, 4096, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=1,KP=2,NS=4>"      # n < 4096
    assert kn(A, 32, 4096, 4608, fw.BF16, X, Q) == "seg_kernel<SEG=1,T=2,W=4,U=1,MT=2>"     # k % 2048 != 0
    assert kn(A, 3, 14336, 4096, fw.BF16, X, Q) == "pipe_kernel<XR=4,CT=4,KP=1,NS=4>"
    assert kn(A, 8, 4096, 4096, fw.BF16, X, Q) == "narrow_kernel<MT=1,W=4,NS=4>"
    assert kn(A, 4, 4096, 2048, fw.BF16, X, Q) == "seg_kernel<SEG=4,T=4,W=4,U=2,MT=1>"
    assert kn(A, 8, 4096, 2048, fw.BF16, X, Q) == "seg_kernel<SEG=2,T=2,W=8,U=2,MT=1>"
    assert kn(A, 12, 40, 768, fw.BF16, X, Q) == "seg_kernel<SEG=1,T=2,W=4,U=1,MT=2>"      # k % 1024 != 0
    assert kn(A, 12, 40, 1024, fw.BF16, X, Q) == "pipe_kernel<XR=12,CT=1,KP=2,NS=2>"
    assert kn(A, 13, 40, 1024, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=1,KP=2,NS=2>"
    assert kn(A, 20, 12300, 512, fw.BF16, X, Q) == "pipe_kernel<XR=24,CT=4,KP=1,NS=2>"
    assert kn(A, 16, 12288, 4096, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=3,KP=1,NS=4>"
    assert kn(fw.PATH_SKINNY, 1, 4096, 4096, fw.BF16, X, Q) == "seg_kernel<SEG=4,T=4,W=4,U=2,MT=1>"
    assert kn(A, 4, 28672, 8200, fw.BF16, X, Q) == "pipe_kernel<XR=4,CT=4,KP=1,NS=2,CB=8>"
    assert kn(A, 1, 28672, 8200, fw.BF16, X, Q) == "gemv_shift_kernel<R=4,U=2,NT=128>"  # k % 16 == 8
    assert kn(A, 1, 4096, 4104, fw.BF16, X, Q) == "gemv_shift_kernel<R=2,U=2,NT=64,DB>"
    assert kn(A, 1, 4096, 4096, fw.BF16, X, Q + 8) == "gemv_kernel<R=2,U=2,NT=64,DB,CH=8>"  # every row 8 bytes off
    assert kn(A, 1, 28672, 8192, fw.BF16, X, Q + 8) == "gemv_kernel<R=4,U=2,NT=128,CH=8>"
    assert kn(A, 1, 4096, 4112, fw.BF16, X, Q) == "gemv_kernel<R=2,U=2,NT=64,DB>"   # k % 16 == 0: 16-code chunks
    assert kn(A, 1, 28672, 8200, fw.BF16, X, Q + 4) == "pipe_kernel<XR=4,CT=4,KP=1,NS=2,CB=4>"
    assert kn(A, 4, 4096, 14344, fw.BF16, X, Q) == "pipe_kernel<XR=4,CT=1,KP=2,NS=4,CB=8>"
    assert kn(A, 32, 28672, 8200, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=4,KP=1,NS=2,CB=8>"
    assert kn(A, 16, 14336, 4104, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=4,KP=1,NS=4,CB=8>"
    assert kn(A, 16, 4096, 4096, fw.BF16, X, Q + 4) == "pipe_kernel<XR=16,CT=1,KP=2,NS=4,CB=4>"
    assert kn(A, 9, 100, 776, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=2,KP=1,NS=2,CB=8>"   # 768 = 3 stages: 512
    assert kn(A, 32, 2048, 4096 + 8, fw.BF16, X, Q) == "pipe_kernel<XR=32,CT=1,KP=2,NS=2,CB=8>"
    # every row 8 bytes off a 16-byte boundary (k % 16 == 0, q 8 bytes off): 4-byte loads
    assert kn(A, 8, 4096, 4096, fw.BF16, X, Q + 8) == "pipe_kernel<XR=8,CT=1,KP=2,NS=4,CB=4>"
    assert kn(A, 16, 8192, 4112, fw.BF16, X, Q) == "pipe_kernel<XR=16,CT=2,KP=2,NS=4,CB=8>"  # aligned rows
    assert kn(fw.PATH_FALLBACK, 4, 28672, 8200, fw.BF16, X, Q) == "dequantize_kernel+wpipe_kernel<XR=4,CT=4,NS=4>"
    assert kn(A, 40, 300, 1000, fw.FP16, X, Q) == "dequantize_kernel+wpipe_kernel<XR=32,CT=4,NS=4>"
    assert kn(A, 5, 31, 37, fw.BF16, X, Q) == "dequantize_kernel+fallback_gemm_kernel"       # k % 8 != 0
    assert kn(A, 4, 128, 200, fw.BF16, X, Q) == "dequantize_kernel+fallback_gemm_kernel"     # k < 256
    assert kn(A, 3, 100, 4096, fw.BF16, X + 2, Q) == "dequantize_kernel+fallback_gemm_kernel"  # x unaligned
    assert kn(fw.PATH_GEMV, 2, 4096, 4096, fw.BF16, X, Q) is None
    assert kn(fw.PATH_SKINNY, 33, 4096, 4096, fw.BF16, X, Q) is None
    assert kn(A, 33, 4096, 4096, fw.BF16, X, Q) == "batch_kernel<BN=64,BM=64,W=4>x4+splitk_reduce_kernel"
    assert kn(A, 64, 14336, 4096, fw.BF16, X, Q) == "batch_kernel<BN=128,BM=64,W=8>x2+splitk_reduce_kernel"
    assert kn(A, 128, 14336, 4096, fw.BF16, X, Q) == "batch_kernel<BN=128,BM=64,W=8>"
    assert kn(A, 128, 4096, 4096, fw.BF16, X, Q) == "batch_kernel<BN=128,BM=64,W=8>x4+splitk_reduce_kernel"
    assert kn(A, 512, 14336, 4096, fw.BF16, X, Q) == "batch_kernel<BN=256,BM=128,W=8>"
    assert kn(A, 2048, 14336, 4096, fw.BF16, X, Q) == "batch_kernel<BN=256,BM=128,W=8>"
    assert kn(A, 33, 64, 256, fw.BF16, X, Q) == "batch_kernel<BN=32,BM=32,W=1>"
    assert kn(fw.PATH_BATCH, 1, 4096, 4096, fw.BF16, X, Q) == "batch_kernel<BN=32,BM=32,W=1>"  # no workspace
    assert kn(fw.PATH_BATCH, 64, 4096, 4100, fw.BF16, X, Q) is None     # k % 256 != 0
    assert kn(A, 1, 4096, 4096, fw.FP32, X, Q) is None
    assert kn(7, 1, 4096, 4096, fw.BF16, X, Q) is None


def test_workspace_bytes():
    wb = fw.fp8w_linear_workspace_bytes
    assert wb(1, 4096, 4096, fw.BF16, X, Q, Y) == 0
    assert wb(16, 4096, 4096, fw.BF16, X, Q, Y) == 0
    assert wb(4, 28672, 8200, fw.BF16, X, Q, Y) == 0                     # 4-byte skinny path
    assert wb(4, 28672, 8196, fw.BF16, X, Q, Y) == 28672 * 8196 * 2      # k % 8 != 0: fallback
    assert wb(32, 4096, 14336, fw.BF16, X, Q + 4, Y) == 0                 # unaligned-code path: no split
    assert wb(64, 100, 500, fw.FP16, X, Q, Y) == 100 * 500 * 2           # k % 256 != 0: fallback
    assert wb(64, 100, 512, fw.FP16, X, Q, Y) == 0                       # batch kernel, single pass
    assert wb(64, 14336, 4096, fw.BF16, X, Q, Y) == 2 * 64 * 14336 * 4    # batch kernel, k in two
    assert wb(512, 14336, 4096, fw.BF16, X, Q, Y) == 0
    assert wb(1, 10, 0, fw.BF16, X, Q, Y) == 0
    assert wb(1, 4096, 4096, fw.FP32, X, Q, Y) == 0
    assert wb(32, 8192, 28672, fw.BF16, X, Q, Y) == 2 * 32 * 8192 * 4     # split k
    assert wb(17, 11000, 4096, fw.FP16, X, Q, Y) == 2 * 17 * 11000 * 4
    assert wb(16, 8192, 28672, fw.BF16, X, Q, Y) == 2 * 16 * 8192 * 4     # split k from 12 tokens on long rows
    assert wb(11, 8192, 28672, fw.BF16, X, Q, Y) == 0
    assert wb(16, 8192, 14336, fw.BF16, X, Q, Y) == 0
    assert wb(32, 4096, 14336, fw.BF16, X, Q, Y) == 4 * 32 * 4096 * 4    # split k in four
    assert wb(16, 4096, 14336, fw.BF16, X, Q, Y) == 4 * 16 * 4096 * 4    # split k in four from 12 tokens
    assert wb(11, 4096, 14336, fw.BF16, X, Q, Y) == 0
    assert wb(16, 4096, 11008, fw.BF16, X, Q, Y) == 4 * 16 * 4096 * 4    # odd stage count: uneven split in four
    assert wb(8, 4096, 11008, fw.BF16, X, Q, Y) == 0
    assert wb(32, 8192, 1024, fw.BF16, X, Q, Y) == 0                      # k % 2048 != 0


def test_workspace_bytes_per_path():
    """The per-path query: auto equals fp8w_linear_workspace_bytes; a forced fallback
    always needs the 16-bit weight; a forced skinny or batch path splits k (and uses
    workspace) only where it is also the automatic path."""
    pw = fw.fp8w_linear_with_path_workspace_bytes
    wb = fw.fp8w_linear_workspace_bytes
    for (m, n, k, act) in [(1, 4096, 4096, fw.BF16), (32, 4096, 14336, fw.BF16), (4, 28672, 8200, fw.BF16),
                           (64, 14336, 4096, fw.BF16), (17, 11000, 4096, fw.FP16), (64, 100, 500, fw.FP16)]:
        assert pw(fw.PATH_AUTO, m, n, k, act, X, Q) == wb(m, n, k, act, X, Q, Y)
    assert pw(fw.PATH_FALLBACK, 1, 4096, 4096, fw.BF16, X, Q) == 4096 * 4096 * 2
    assert pw(fw.PATH_FALLBACK, 32, 4096, 14336, fw.FP16, X, Q) == 4096 * 14336 * 2
    assert pw(fw.PATH_SKINNY, 32, 4096, 14336, fw.BF16, X, Q) == 4 * 32 * 4096 * 4
    assert pw(fw.PATH_BATCH, 32, 4096, 14336, fw.BF16, X, Q) == 0      # forced: single pass
    assert pw(fw.PATH_SKINNY, 1, 4096, 4096, fw.BF16, X, Q) == 0
    assert pw(fw.PATH_BATCH, 64, 14336, 4096, fw.BF16, X, Q) == 2 * 64 * 14336 * 4
    assert pw(fw.PATH_GEMV, 1, 4096, 4096, fw.BF16, X, Q) == 0
    assert pw(7, 1, 4096, 4096, fw.BF16, X, Q) == 0
    assert pw(fw.PATH_FALLBACK, 1, 4096, 4096, fw.FP32, X, Q) == 0   # invalid activation dtype


def _lin(x=X, act=fw.BF16, m=4, k=4096, q=Q, s=S, b=B, n=4096, y=Y, ws=0, wsb=0, path=fw.PATH_AUTO):
    return fw.fp8w_linear_with_path(x, act, m, k, q, s, b, n, y, ws, wsb, path, 0)


def test_linear_rejects_invalid_arguments():
    assert _lin(act=fw.FP32) == fw.ERR_INVALID_VALUE
    assert _lin(act=7) == fw.ERR_INVALID_VALUE
    assert _lin(m=-1) == fw.ERR_INVALID_VALUE
    assert _lin(n=-1) == fw.ERR_INVALID_VALUE
    assert _lin(k=-256) == fw.ERR_INVALID_VALUE
    assert _lin(m=2_000_000) == fw.ERR_INVALID_VALUE
    assert _lin(x=0) == fw.ERR_INVALID_VALUE
    assert _lin(q=0) == fw.ERR_INVALID_VALUE
    assert _lin(s=0) == fw.ERR_INVALID_VALUE
    assert _lin(y=0) == fw.ERR_INVALID_VALUE
    assert _lin(s=S + 2) == fw.ERR_MISALIGNED
    assert _lin(b=B + 1) == fw.ERR_MISALIGNED
    assert _lin(y=Y + 1) == fw.ERR_MISALIGNED
    assert _lin(path=4) == fw.ERR_INVALID_VALUE
    assert _lin(path=-2) == fw.ERR_INVALID_VALUE
    # forced paths the shape cannot take
    assert _lin(m=2, path=fw.PATH_GEMV) == fw.ERR_INVALID_VALUE
    assert _lin(m=33, path=fw.PATH_SKINNY) == fw.ERR_INVALID_VALUE
    assert _lin(k=4004, path=fw.PATH_SKINNY) == fw.ERR_INVALID_VALUE     # k % 8 != 0
    assert _lin(k=504, path=fw.PATH_SKINNY) == fw.ERR_INVALID_VALUE      # unaligned-code path: k >= 512
    assert _lin(k=4104, x=X + 8, path=fw.PATH_SKINNY) == fw.ERR_MISALIGNED  # unaligned-code path: x 16-byte aligned
    assert _lin(q=Q + 2, path=fw.PATH_SKINNY) == fw.ERR_MISALIGNED      # codes at least 4-byte aligned
    assert _lin(k=256, q=Q + 4, path=fw.PATH_SKINNY) == fw.ERR_MISALIGNED  # unaligned-code path needs k >= 512
    assert _lin(m=1, k=4100, path=fw.PATH_GEMV) == fw.ERR_INVALID_VALUE     # k % 8 != 0
    assert _lin(m=1, k=4104, q=Q + 4, path=fw.PATH_GEMV) == fw.ERR_MISALIGNED  # 8-code chunks: q 8-byte aligned
    assert _lin(m=1, k=4104, x=X + 8, path=fw.PATH_GEMV) == fw.ERR_MISALIGNED  # x 16-byte aligned
    assert _lin(m=1, x=X + 2, path=fw.PATH_GEMV) == fw.ERR_MISALIGNED
    assert _lin(m=64, k=4000, path=fw.PATH_BATCH) == fw.ERR_INVALID_VALUE
    assert _lin(m=64, k=128, path=fw.PATH_BATCH) == fw.ERR_INVALID_VALUE
    assert _lin(m=64, q=Q + 8, path=fw.PATH_BATCH) == fw.ERR_MISALIGNED
    assert _lin(m=64, x=X + 2, path=fw.PATH_BATCH) == fw.ERR_MISALIGNED
    assert _lin(m=64, y=X + 64, path=fw.PATH_BATCH) == fw.ERR_INVALID_VALUE
    # y overlapping an input
    assert _lin(y=X + 64) == fw.ERR_INVALID_VALUE
    assert _lin(y=Q) == fw.ERR_INVALID_VALUE
    assert _lin(y=S - 16) == fw.ERR_INVALID_VALUE
    assert _lin(y=B) == fw.ERR_INVALID_VALUE


def test_split_k_workspace_is_validated():
    need = 2 * 32 * 8192 * 4
    big = dict(m=32, n=8192, k=28672)
    assert _lin(ws=WS + 8, wsb=need, **big) == fw.ERR_MISALIGNED
    assert _lin(ws=X, wsb=need, **big) == fw.ERR_INVALID_VALUE      # overlaps x
    assert _lin(ws=Y - 64, wsb=need, **big) == fw.ERR_INVALID_VALUE  # overlaps y


def test_batch_split_workspace_is_validated():
    need = 2 * 64 * 14336 * 4
    big = dict(m=64, n=14336, k=4096)
    assert _lin(ws=WS + 8, wsb=need, **big) == fw.ERR_MISALIGNED
    assert _lin(ws=X, wsb=need, **big) == fw.ERR_INVALID_VALUE      # overlaps x
    assert _lin(ws=Y - 64, wsb=need, **big) == fw.ERR_INVALID_VALUE  # overlaps y


def test_linear_fallback_needs_workspace():
    assert _lin(k=8200, path=fw.PATH_FALLBACK) == fw.ERR_WORKSPACE
    assert _lin(k=8196) == fw.ERR_WORKSPACE                               # k % 8 != 0: the fallback
    assert _lin(k=8200, ws=WS, wsb=4096 * 8200 * 2 - 1, path=fw.PATH_FALLBACK) == fw.ERR_WORKSPACE
    assert _lin(k=8196, ws=WS + 1, wsb=4096 * 8196 * 2) == fw.ERR_MISALIGNED
    assert _lin(k=8196, ws=X, wsb=4096 * 8196 * 2) == fw.ERR_INVALID_VALUE  # overlaps x
    assert _lin(m=64, path=fw.PATH_FALLBACK) == fw.ERR_WORKSPACE


def test_zero_sized_calls_succeed_without_a_device():
    assert _lin(m=0) == fw.SUCCESS
    assert _lin(n=0) == fw.SUCCESS
    assert _lin(m=0, x=0, y=0) == fw.SUCCESS
    assert _lin(m=0, path=fw.PATH_BATCH) == fw.SUCCESS
    assert _lin(m=64, n=0, path=fw.PATH_BATCH) == fw.SUCCESS
    assert fw.fp8w_quantize(0, fw.FP32, 0, 100, 0, 0, 0) == fw.SUCCESS
    assert fw.fp8w_dequantize_fallback(0, 0, 0, 100, 0, fw.BF16, 0) == fw.SUCCESS
    assert fw.fp8w_dequantize_fallback(Q, S, 100, 0, 0, fw.BF16, 0) == fw.SUCCESS


def test_quantize_rejects_invalid_arguments():
    qz = fw.fp8w_quantize
    assert qz(X, 9, 10, 10, Q, S, 0) == fw.ERR_INVALID_VALUE
    assert qz(X, fw.FP32, -1, 10, Q, S, 0) == fw.ERR_INVALID_VALUE
    assert qz(X, fw.FP32, 10, -1, Q, S, 0) == fw.ERR_INVALID_VALUE
    assert qz(0, fw.FP32, 10, 10, Q, S, 0) == fw.ERR_INVALID_VALUE
    assert qz(X, fw.FP32, 10, 10, 0, S, 0) == fw.ERR_INVALID_VALUE
    assert qz(X, fw.FP32, 10, 10, Q, 0, 0) == fw.ERR_INVALID_VALUE
    assert qz(X + 2, fw.FP32, 10, 10, Q, S, 0) == fw.ERR_MISALIGNED
    assert qz(X, fw.FP32, 10, 10, Q, S + 1, 0) == fw.ERR_MISALIGNED
    assert qz(X, fw.FP32, 10, 10, X + 16, S, 0) == fw.ERR_INVALID_VALUE  # q overlaps w
    assert qz(X, fw.FP32, 10, 10, Q, X, 0) == fw.ERR_INVALID_VALUE       # scale overlaps w
    assert qz(X, fw.FP32, 1 << 31, 10, Q, S, 0) == fw.ERR_INVALID_VALUE


def test_read_probe_rejects_invalid_arguments():
    rp = fw.fp8w_stream_read_probe
    assert rp(X, 0, S, 0) == fw.SUCCESS
    assert rp(0, 4096, S, 0) == fw.ERR_INVALID_VALUE
    assert rp(X, 4096, 0, 0) == fw.ERR_INVALID_VALUE
    assert rp(X, 4095, S, 0) == fw.ERR_INVALID_VALUE
    assert rp(X + 8, 4096, S, 0) == fw.ERR_MISALIGNED


def test_dequantize_rejects_invalid_arguments():
    dq = fw.fp8w_dequantize_fallback
    assert dq(Q, S, 10, 10, Y, 5, 0) == fw.ERR_INVALID_VALUE
    assert dq(0, S, 10, 10, Y, fw.BF16, 0) == fw.ERR_INVALID_VALUE
    assert dq(Q, S, 10, 10, 0, fw.BF16, 0) == fw.ERR_INVALID_VALUE
    assert dq(Q, S, 10, 10, Y + 2, fw.FP32, 0) == fw.ERR_MISALIGNED
    assert dq(Q, S + 2, 10, 10, Y, fw.FP32, 0) == fw.ERR_MISALIGNED
    assert dq(Q, S, 10, 10, Q + 4, fw.BF16, 0) == fw.ERR_INVALID_VALUE  # out overlaps q


def test_product_path_fails_loudly_without_the_library(tmp_path, monkeypatch):
    """With libfp8w.so absent there is no fallback: every entry point raises."""
    monkeypatch.setattr(fw, "_LIB", None)
    monkeypatch.setattr(fw, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fw.fp8w_abi_version()
    with pytest.raises(RuntimeError, match="missing"):
        fw.fp8w_linear_path(1, 1, 256, fw.BF16, 0, 0, 0)


def test_package_never_imports_the_oracle():
    import subprocess
    import sys
    code = ("import sys; import fp8_weight_only_amd; "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), 'oracle imported'")
    subprocess.run([sys.executable, "-c", code], cwd=ROOT, check=True)
    for dirpath, _, files in os.walk(os.path.join(ROOT, "fp8_weight_only_amd")):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                with open(os.path.join(dirpath, f)) as fh:
                    text = fh.read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "fp8w_oracle" not in text and "liboracle" not in text, f


# ---------------------------------------------------------------- group scales
def _glin(x=X, act=fw.BF16, m=4, k=4096, q=Q, s=S, g=32, b=B, n=4096, y=Y, path=fw.PATH_AUTO):
    return fw.fp8w_linear_grouped_with_path(x, act, m, k, q, s, g, b, n, y, path, 0)


def test_grouped_paths_and_kernel_names():
    gp, gk, A = fw.fp8w_linear_grouped_path, fw.fp8w_linear_grouped_kernel, fw.PATH_AUTO
    assert gp(1, 4096, 4096, 32, fw.BF16, X, Q) == fw.PATH_GEMV
    assert gp(16, 4096, 4096, 64, fw.BF16, X, Q) == fw.PATH_SKINNY
    assert gp(33, 4096, 4096, 128, fw.BF16, X, Q) == fw.PATH_BATCH
    assert gp(33, 4096, 4160, 64, fw.BF16, X, Q) == fw.PATH_FALLBACK     # k % 256 != 0
    assert gp(33, 4096, 4096, 64, fw.BF16, X + 2, Q) == fw.PATH_FALLBACK  # x not 16-byte aligned
    assert gp(1, 4096, 4160, 32, fw.BF16, X, Q) == fw.PATH_FALLBACK      # k % 256 != 0
    assert gp(1, 4096, 4096, 48, fw.BF16, X, Q) == -1                    # group not 32/64/128
    assert gp(1, 4096, 4000, 64, fw.BF16, X, Q) == -1                    # group does not divide k
    assert gk(A, 1, 4096, 4096, 32, fw.BF16, X, Q) == "gemv_grouped_kernel<R=2,U=2,NT=64,DB>"
    assert gk(A, 1, 28672, 8192, 128, fw.BF16, X, Q) == "gemv_grouped_kernel<R=4,U=2,NT=128>"
    assert gk(A, 16, 14336, 4096, 32, fw.FP16, X, Q) == "pipe_grouped_kernel<XR=16,CT=4,KP=1,NS=4>"
    assert gk(A, 32, 28672, 4096, 32, fw.BF16, X, Q) == "pipe_grouped_kernel<XR=32,CT=4,KP=1,NS=2>"
    assert gk(A, 8, 4096, 4096, 64, fw.BF16, X, Q) == "pipe_grouped_kernel<XR=8,CT=1,KP=2,NS=4>"
    assert gk(A, 32, 4096, 4096, 64, fw.BF16, X, Q) == "pipe_grouped_kernel<XR=32,CT=1,KP=2,NS=2>"
    assert gk(A, 2, 4096, 768, 128, fw.BF16, X, Q) == "grouped_generic_kernel"      # ring cannot tile k
    assert gk(A, 64, 4096, 4096, 32, fw.BF16, X, Q) == "batch_grouped_kernel<BN=64,BM=64,W=4>x4+splitk_reduce_kernel"
    assert gk(A, 128, 14336, 4096, 128, fw.BF16, X, Q) == "batch_grouped_kernel<BN=128,BM=64,W=8>"
    assert gk(A, 128, 14336, 4096, 32, fw.BF16, X, Q).startswith("batch_grouped_kernel<BN=64,")  # no 128 x 64 for g 32
    assert gk(fw.PATH_BATCH, 2, 4096, 4096, 64, fw.BF16, X, Q) == "batch_grouped_kernel<BN=64,BM=32,W=2>"
    assert gk(fw.PATH_BATCH, 40, 4096, 4160, 64, fw.BF16, X, Q) is None    # k % 256 != 0
    assert gk(A, 64, 4096, 4160, 64, fw.BF16, X, Q) == "grouped_generic_kernel"
    assert gk(fw.PATH_FALLBACK, 1, 4096, 4096, 32, fw.BF16, X, Q) == "grouped_generic_kernel"
    assert gk(fw.PATH_GEMV, 2, 4096, 4096, 32, fw.BF16, X, Q) is None


def test_grouped_workspace_bytes_and_validation():
    wb = fw.fp8w_linear_grouped_workspace_bytes
    assert wb(64, 4096, 4096, 32, fw.BF16, X, Q) == 4 * 64 * 4096 * 4              # x4 split
    assert wb(300, 4096, 4096, 64, fw.BF16, X, Q) == 0                             # single pass
    assert wb(16, 4096, 4096, 32, fw.BF16, X, Q) == 0                              # skinny path
    assert wb(64, 4096, 4160, 64, fw.BF16, X, Q) == 0                              # generic kernel
    assert wb(64, 4096, 4096, 48, fw.BF16, X, Q) == 0                              # invalid group

    def g(ws, nbytes, **kw):
        a = dict(x=X, act=fw.BF16, m=64, k=4096, q=Q, s=S, g=32, b=B, n=4096, y=Y, path=fw.PATH_AUTO)
        a.update(kw)
        return fw.fp8w_linear_grouped_with_workspace(a["x"], a["act"], a["m"], a["k"], a["q"], a["s"], a["g"],
                                                     a["b"], a["n"], a["y"], ws, nbytes, a["path"], 0)
    need = wb(64, 4096, 4096, 32, fw.BF16, X, Q)
    assert g(WS + 8, need) == fw.ERR_MISALIGNED                                   # used, not 16-byte aligned
    assert g(Y, need) == fw.ERR_INVALID_VALUE                                     # overlaps y
    assert g(0, 0, m=0) == fw.SUCCESS
    assert g(WS, need, path=4) == fw.ERR_INVALID_VALUE


def test_grouped_rejects_invalid_arguments():
    assert _glin(g=16) == fw.ERR_INVALID_VALUE
    assert _glin(g=256) == fw.ERR_INVALID_VALUE
    assert _glin(k=4000, g=64) == fw.ERR_INVALID_VALUE
    assert _glin(act=fw.FP32) == fw.ERR_INVALID_VALUE
    assert _glin(s=S + 2) == fw.ERR_MISALIGNED
    assert _glin(x=X + 2, path=fw.PATH_SKINNY) == fw.ERR_MISALIGNED
    assert _glin(m=2, path=fw.PATH_GEMV) == fw.ERR_INVALID_VALUE
    assert _glin(k=4160, path=fw.PATH_SKINNY) == fw.ERR_INVALID_VALUE
    assert _glin(y=Q) == fw.ERR_INVALID_VALUE                            # y overlaps q
    assert _glin(path=5) == fw.ERR_INVALID_VALUE
    assert _glin(path=4) == fw.ERR_INVALID_VALUE
    assert _glin(m=40, k=4160, path=fw.PATH_BATCH) == fw.ERR_INVALID_VALUE
    assert _glin(m=40, x=X + 2, path=fw.PATH_BATCH) == fw.ERR_MISALIGNED
    assert _glin(m=0) == fw.SUCCESS
    assert _glin(n=0) == fw.SUCCESS


def test_grouped_quantize_and_dequantize_validation():
    qg, dg = fw.fp8w_quantize_grouped, fw.fp8w_dequantize_grouped
    assert qg(0, fw.FP32, 0, 64, 32, 0, 0, 0) == fw.SUCCESS
    assert qg(X, fw.FP32, 4, 64, 48, Q, S, 0) == fw.ERR_INVALID_VALUE
    assert qg(X, fw.FP32, 4, 96, 64, Q, S, 0) == fw.ERR_INVALID_VALUE
    assert qg(X + 2, fw.FP32, 4, 64, 32, Q, S, 0) == fw.ERR_MISALIGNED
    assert qg(X, fw.FP32, 4, 64, 32, Q, 0, 0) == fw.ERR_INVALID_VALUE
    assert dg(Q, S, 32, 0, 64, Y, fw.BF16, 0) == fw.SUCCESS
    assert dg(Q, 0, 32, 4, 64, Y, fw.BF16, 0) == fw.ERR_INVALID_VALUE
    assert dg(Q, S, 32, 4, 64, Y + 1, fw.BF16, 0) == fw.ERR_MISALIGNED
    assert dg(Q, S, 32, 4, 64, Q, fw.BF16, 0) == fw.ERR_INVALID_VALUE    # out overlaps q


def test_fnuz_to_ocp_validation():
    f = fw.fp8w_fnuz_to_ocp
    assert f(0, 0, 0, 0) == fw.SUCCESS
    assert f(Q, -1, Y, 0) == fw.ERR_INVALID_VALUE
    assert f(0, 16, Y, 0) == fw.ERR_INVALID_VALUE
    assert f(Q, 64, Q + 8, 0) == fw.ERR_INVALID_VALUE     # partial overlap


def test_w8a8_validation():
    g = fw.fp8w_gemm_w8a8
    assert g(X, S, 0, 4096, Q, S, 0, 4096, Y, fw.BF16, 0) == fw.SUCCESS
    assert g(X, S, 64, 4000, Q, S, 0, 4096, Y, fw.BF16, 0) == fw.ERR_INVALID_VALUE    # k % 256 != 0
    assert g(X, S, 64, 4096, Q, S, 0, 4096, Y, fw.FP32, 0) == fw.ERR_INVALID_VALUE
    assert g(X + 8, S, 64, 4096, Q, S, 0, 4096, Y, fw.BF16, 0) == fw.ERR_MISALIGNED
    assert g(X, S, 64, 4096, Q, S, 0, 4096, Q, fw.BF16, 0) == fw.ERR_INVALID_VALUE    # y overlaps q
    assert fw.fp8w_linear_w8a8_workspace_bytes(100, 256) == 25600 + 400
    assert fw.fp8w_linear_w8a8_workspace_bytes(3, 256) == 768 + 12
    lw = fw.fp8w_linear_w8a8
    assert lw(X, fw.BF16, 64, 4096, Q, S, 0, 4096, Y, 0, 0, 0) == fw.ERR_WORKSPACE
    assert lw(X, fw.BF16, 64, 4096, Q, S, 0, 4096, Y, WS + 8, 1 << 22, 0) == fw.ERR_MISALIGNED
    assert lw(X, fw.BF16, 64, 4096, Q, S, 0, 4096, Y, X, 1 << 22, 0) == fw.ERR_INVALID_VALUE  # overlaps x
    # the GEMM's arguments are checked before the activation quantizer is enqueued
    assert lw(X, fw.BF16, 64, 4096, 0, S, 0, 4096, Y, WS, 1 << 22, 0) == fw.ERR_INVALID_VALUE     # no weight codes
    assert lw(X, fw.BF16, 64, 4096, Q, 0, 0, 4096, Y, WS, 1 << 22, 0) == fw.ERR_INVALID_VALUE     # no weight scales
    assert lw(X, fw.BF16, 64, 4096, Q + 8, S, 0, 4096, Y, WS, 1 << 22, 0) == fw.ERR_MISALIGNED
    assert lw(X, fw.BF16, 64, 4096, Q, S + 2, 0, 4096, Y, WS, 1 << 22, 0) == fw.ERR_MISALIGNED
    assert lw(X, fw.BF16, 64, 4096, Q, S, 0, 4096, Q, WS, 1 << 22, 0) == fw.ERR_INVALID_VALUE     # y overlaps q
    assert fw.fp8w_quantize_activations(X, fw.BF16, 0, 64, Q, S, 0) == fw.SUCCESS
    assert fw.fp8w_quantize_activations(X, fw.FP32, 4, 64, Q, S, 0) == fw.ERR_INVALID_VALUE
    assert fw.fp8w_linear_w8a8_kernel(4096, 4096, 4096) == "w8a8_kernel<BN=256,BM=256,NS=4,W=8>"
    assert fw.fp8w_linear_w8a8_kernel(2048, 4096, 4096) == "w8a8_kernel<BN=256,BM=128,NS=4,W=8>"
    assert fw.fp8w_linear_w8a8_kernel(1024, 4096, 4096) == "w8a8_kernel<BN=128,BM=128,NS=4,W=8>"
    assert fw.fp8w_linear_w8a8_kernel(500, 4000, 1536) == "w8a8_kernel<BN=128,BM=64,NS=8,W=4>"     # 256 tiles
    assert fw.fp8w_linear_w8a8_kernel(500, 4000, 768) == "w8a8_kernel<BN=128,BM=64,NS=4,W=4>"      # k % 512 != 0
    assert fw.fp8w_linear_w8a8_kernel(700, 4000, 1536) == "w8a8_kernel<BN=128,BM=64,NS=4,W=4>"     # 352 tiles
    assert fw.fp8w_linear_w8a8_kernel(512, 4096, 4096) == "w8a8_kernel<BN=128,BM=64,NS=8,W=4>"
    assert fw.fp8w_linear_w8a8_kernel(100, 200, 256) == "w8a8_kernel<BN=128,BM=64,NS=4,W=4>"
    assert fw.fp8w_linear_w8a8_kernel(512, 14336, 4096) == "w8a8_kernel<BN=256,BM=128,NS=4,W=8>"
    assert fw.fp8w_linear_w8a8_kernel(512, 4096, 4000) is None


def test_noalloc_rejects_before_touching_the_gpu():
    """fp8w_linear_noalloc validates like fp8w_linear, and a fallback call whose
    16-bit weight would not fit the static scratch is refused before any HIP call
    (so these run without a GPU)."""
    na = fw.fp8w_linear_noalloc
    assert fw.SCRATCH_BYTES == 32 << 20
    # k % 8 != 0: the fallback; 28672 x 8196 x 2 bytes > 32 MiB
    assert na(X, fw.BF16, 4, 8196, Q, S, 0, 28672, Y, 0) == fw.ERR_WORKSPACE
    # misaligned x: the fallback too, 4096 x 4096 x 2 = exactly 32 MiB would fit, 4097 rows do not
    assert na(X + 2, fw.BF16, 4, 4096, Q, S, 0, 4097, Y, 0) == fw.ERR_WORKSPACE
    assert na(X, fw.FP32, 4, 4096, Q, S, 0, 4096, Y, 0) == fw.ERR_INVALID_VALUE
    assert na(X, fw.BF16, 4, 4096, Q, 0, 0, 4096, Y, 0) == fw.ERR_INVALID_VALUE      # no scale
    assert na(X, fw.BF16, 4, 4096, Q, S, 0, 4096, X, 0) == fw.ERR_INVALID_VALUE      # y overlaps x
    assert na(X, fw.BF16, 0, 4096, Q, S, 0, 4096, Y, 0) == fw.SUCCESS                # empty: nothing runs
