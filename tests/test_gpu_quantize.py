"""GPU parity of the build-time quantizer (fp8w_quantize) against the oracle:
scales and codes must be bit-identical.

Sources: "FP8 weight-only (precision: fp8_weights)", section "The contract";
"Skill: Write an FP8 Kernel", "Required reasoning process" steps 2, 4 and 7.
"""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_same_bits

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(w_np: np.ndarray, dtype=torch.float32):
    w_t = torch.from_numpy(w_np).to(dtype)
    w_ref = w_t.float().numpy()  # exact widening of bf16 / fp16 weights
    q, s = fw.quantize(w_t.to(DEV))
    torch.cuda.synchronize()
    q_ref, s_ref, st = oracle.quantize_rows(w_ref)
    assert st == 0
    return q.cpu().numpy(), s.cpu().numpy(), q_ref, s_ref


@pytest.mark.parametrize("shape", [(1, 1), (3, 17), (16, 256), (33, 1000), (64, 4096), (5, 8200), (7, 255),
                                   (2, 4097), (1, 65536)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
def test_quantize_shapes_bitexact(shape, dtype):
    print(f"quantize shape={shape} dtype={dtype}", flush=True)
    g = np.random.default_rng(hash(shape) % 1000)
    w = (g.standard_normal(shape) * 0.02).astype(np.float32)
    q, s, q_ref, s_ref = _run(w, dtype)
    assert_same_bits(s, s_ref, "scale")
    assert_same_bits(q, q_ref, "codes")


def test_quantize_special_rows_bitexact():
    """Zero rows, signed zeros, subnormal and huge magnitudes, a scale that
    underflows to 0, rows that hit the +-448 clamp, exact ties."""
    k = 1024
    rows = []
    g = np.random.default_rng(1)
    rows.append(np.zeros(k))                                           # scale 0
    rows.append(np.where(np.arange(k) % 2, -0.0, 0.0))                 # signed zeros
    rows.append(g.standard_normal(k) * 1e-40)                          # subnormal weights / scale
    rows.append(g.standard_normal(k) * 1e-44)                          # scale underflows to 0
    rows.append(g.standard_normal(k) * 3e37)                           # huge
    rows.append(np.concatenate([[3.0e38], g.standard_normal(k - 1)]))  # one huge outlier
    r = np.concatenate([[448.0], oracle.decode(np.arange(0x7F)), -oracle.decode(np.arange(0x7F))])
    mids = 0.5 * (oracle.decode(np.arange(1, 0x7F)) + oracle.decode(np.arange(0, 0x7E)))
    r = np.concatenate([r, mids, -mids])
    rows.append(np.resize(r, k))                                       # every code and every tie
    rows.append(g.standard_t(1.0, k))                                  # heavy tail
    w = np.stack(rows).astype(np.float32)
    q, s, q_ref, s_ref = _run(w)
    assert s_ref[0] == 0.0 and s_ref[3] == 0.0
    assert_same_bits(s, s_ref, "scale")
    assert_same_bits(q, q_ref, "codes")


def test_quantize_nonfinite_rejected():
    w = np.ones((4, 300), dtype=np.float32)
    w[1, 7] = np.nan
    w[3, 0] = -np.inf
    with pytest.raises(fw.Fp8wError) as ei:
        fw.quantize(torch.from_numpy(w).to(DEV))
    assert ei.value.status == fw.ERR_NONFINITE
    # raw call: finite rows are still right, the bad rows' scales are NaN
    wd = torch.from_numpy(w).to(DEV)
    q = torch.empty((4, 300), dtype=torch.uint8, device=DEV)
    s = torch.empty((4,), dtype=torch.float32, device=DEV)
    st = fw.fp8w_quantize(wd.data_ptr(), fw.FP32, 4, 300, q.data_ptr(), s.data_ptr(), 0)
    assert st == fw.ERR_NONFINITE
    sc = s.cpu().numpy()
    assert np.isnan(sc[1]) and np.isnan(sc[3])
    assert sc[0] == np.float32(1.0) / np.float32(448.0)
    assert np.all(q.cpu().numpy()[0] == 0x7E)


def test_quantize_unaligned_pointers_bitexact():
    """Offsets that break 16-byte alignment take the element-wise path."""
    g = np.random.default_rng(2)
    n, k = 9, 640
    w = (g.standard_normal((n, k)) * 0.02).astype(np.float32)
    big = torch.zeros(n * k + 1, dtype=torch.float32, device=DEV)
    big[1:] = torch.from_numpy(w.reshape(-1)).to(DEV)
    qbuf = torch.zeros(n * k + 3, dtype=torch.uint8, device=DEV)
    s = torch.empty(n, dtype=torch.float32, device=DEV)
    st = fw.fp8w_quantize(big.data_ptr() + 4, fw.FP32, n, k, qbuf.data_ptr() + 3, s.data_ptr(), 0)
    assert st == fw.SUCCESS
    q_ref, s_ref, _ = oracle.quantize_rows(w)
    assert_same_bits(s.cpu().numpy(), s_ref, "scale")
    assert_same_bits(qbuf.cpu().numpy()[3:].reshape(n, k), q_ref, "codes")
    assert qbuf[:3].sum().item() == 0


def _pattern_rows(first: int, count: int, k: int = 4096) -> np.ndarray:
    """Rows of k fp32 values: 448.0 in column 0 (so scale == 1 exactly and every
    other element is encoded as itself), then the bit patterns first, first+1, ..."""
    per = k - 1
    rows = -(-count // per)
    pat = np.zeros(rows * per, dtype=np.uint32)
    pat[:count] = np.arange(first, first + count, dtype=np.uint64).astype(np.uint32)
    out = np.empty((rows, k), dtype=np.uint32)
    out[:, 0] = np.float32(448.0).view(np.uint32)
    out[:, 1:] = pat.reshape(rows, per)
    return out.view(np.float32)


@pytest.mark.parametrize("sign", [0, 1])
def test_quantize_exhaustive_fp32_patterns(sign):
    """Every fp32 bit pattern with |w| <= 448 (the quotients the quantizer can
    produce), one sign per test, encoded on the GPU and by the oracle."""
    top = int(np.float32(448.0).view(np.uint32))  # 0x43E00000
    base = sign << 31
    chunk = 1 << 27
    start = 0
    while start <= top:
        cnt = min(chunk, top + 1 - start)
        print(f"exhaustive sign={sign} patterns {base + start:#010x}..{base + start + cnt - 1:#010x}", flush=True)
        w = _pattern_rows(base + start, cnt)
        q, s = fw.quantize(torch.from_numpy(w).to(DEV))
        q = q.cpu().numpy()
        q_ref, s_ref, st = oracle.quantize_rows(w)
        assert st == 0 and np.all(s_ref == 1.0)
        assert np.all(s.cpu().numpy() == 1.0)
        assert_same_bits(q, q_ref, f"codes for patterns from {base + start:#x}")
        start += cnt


def test_quantize_workload_weights():
    """The skinny sweep's Student-t weights and the decoder block's outlier / zero rows."""
    lay = workloads.skinny_layer()
    q, s, q_ref, s_ref = _run(lay.w)
    assert_same_bits(s, s_ref, "scale")
    assert_same_bits(q, q_ref, "codes")
    for i in (0, 4, 6):
        lay = workloads.block_layer(i)
        q, s, q_ref, s_ref = _run(lay.w)
        assert (s_ref == 0).sum() == int(round(0.005 * lay.w.shape[0]))
        assert_same_bits(s, s_ref, "scale")
        assert_same_bits(q, q_ref, "codes")
