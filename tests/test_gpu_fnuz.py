"""GPU carry-over of E4M3FNUZ codes to OCP e4m3fn codes, against the oracle.

Sources: "B04 - Precision & Quantization": the format table's E4M3FNUZ row,
the section "Hardware support, and where the vendors diverge" and the trap
list (the same bits decode a factor of two apart; tag the format).
"""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_gate

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_all_256_codes():
    src = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(DEV)
    got = fw.fnuz_to_ocp(src).cpu().numpy()
    assert np.array_equal(got, oracle.fnuz_to_ocp(np.arange(256, dtype=np.uint8)))


@pytest.mark.parametrize("soff,doff,count", [(0, 0, 1 << 20), (3, 3, 100003), (16, 0, 15), (1, 2, 1),
                                            (5, 7, 4097)])
def test_buffers_with_ragged_heads_and_tails(soff, doff, count):
    """Aligned, equally misaligned (head, 16-byte body, tail) and differently
    misaligned (byte path) source and destination."""
    rng = np.random.default_rng(soff + count)
    host = rng.integers(0, 256, soff + count, dtype=np.uint8)
    buf = torch.from_numpy(host).to(DEV)
    src = buf[soff:]
    out = torch.full((doff + count + 16,), 0xAB, dtype=torch.uint8, device=DEV)
    fw.fnuz_to_ocp(src, out[doff:doff + count])
    o = out.cpu().numpy()
    assert np.array_equal(o[doff:doff + count], oracle.fnuz_to_ocp(host[soff:]))
    assert np.all(o[:doff] == 0xAB) and np.all(o[doff + count:] == 0xAB)   # nothing written outside


def test_in_place_and_dtype_tags():
    rng = np.random.default_rng(5)
    host = rng.integers(0, 256, 4096, dtype=np.uint8)
    t = torch.from_numpy(host).to(DEV)
    fw.fnuz_to_ocp(t, t)
    assert np.array_equal(t.cpu().numpy(), oracle.fnuz_to_ocp(host))
    tagged = torch.from_numpy(host).to(DEV).view(torch.float8_e4m3fnuz)
    assert np.array_equal(fw.ocp_codes(tagged).cpu().numpy(), oracle.fnuz_to_ocp(host))
    ocp = torch.from_numpy(host).to(DEV).view(torch.float8_e4m3fn)
    assert np.array_equal(fw.ocp_codes(ocp).cpu().numpy(), host)


def test_linear_on_a_carried_over_fnuz_checkpoint():
    """A layer quantized the FNUZ way (scale amax / 240, nearest FNUZ code),
    carried over on the GPU and run through fp8w_linear with its scales
    unchanged: the gate against the oracle linear on the carried-over codes,
    and the same gate against the FNUZ reconstruction itself."""
    case = workloads.random_case(77, 8, 300, 1024, torch.bfloat16)
    w = case.layer.w.astype(np.float64)
    s = (np.abs(w).max(axis=1) / 240.0).astype(np.float32)
    vals = oracle.fnuz_decode(np.arange(256, dtype=np.uint8))
    fin = np.flatnonzero(np.isfinite(vals))
    order = np.argsort(vals[fin])
    grid, codes = vals[fin][order], fin[order]
    t = w / s[:, None].astype(np.float64)
    hi = np.clip(np.searchsorted(grid, t), 1, grid.size - 1)
    lo = hi - 1
    pick = np.where(np.abs(grid[hi] - t) < np.abs(t - grid[lo]), hi, lo)   # a nearest FNUZ code
    q_fnuz = codes[pick].astype(np.uint8)
    q = fw.fnuz_to_ocp(torch.from_numpy(q_fnuz).to(DEV))
    q_ref = oracle.fnuz_to_ocp(q_fnuz)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    x = case.x.to(DEV)
    b = case.layer.bias.to(DEV)
    y = fw.linear(x, q, torch.from_numpy(s).to(DEV), b).double().cpu().numpy()
    x64 = case.x.double().numpy()
    b64 = case.layer.bias.double().numpy()
    amax = np.abs(w).max(axis=1)
    assert_gate(y, oracle.linear_f64(x64, q_ref, s, b64), x64, amax, "carried-over codes")
    y_fnuz = x64 @ (vals[q_fnuz] * s[:, None].astype(np.float64)).T + b64
    assert_gate(y, y_fnuz, x64, amax, "FNUZ reconstruction")
