"""Seeded random shapes through every dispatch path of fp8w_linear,
fp8w_linear_grouped and fp8w_linear_w8a8, against the oracle.

Each case draws the number of tokens m, the channels n, the reduction length k
(a multiple of 256, of 16, of 8, of 2, or odd), the activation dtype, a bias or
none, the byte offsets of x, q and y inside larger buffers (which decide the
alignment the dispatcher sees), and whether the caller passes a workspace or an
empty one. Every case checks:
- the path the library reports against the dispatch rule of fp8w_linear in
  include/fp8w.h, restated here;
- every output against the oracle's fp64 value, within the gate of
  tests/parity_util.py ("FP8 weight-only (precision: fp8_weights)", "The
  contract": one fp32 accumulation, scale and bias in fp32, one rounding);
- that nothing is written outside y (guard elements on both sides keep their
  NaN bits) and that x and q are unchanged;
- a fallback call given an empty workspace is refused before any launch and
  leaves y untouched.
The grouped cases draw a group size of 32, 64 or 128 weights along k ("B04 -
Precision & Quantization", "Post-training quantization versus
quantization-aware training") and rows whose groups span three decades in
magnitude, with the same checks against the oracle's grouped linear.
Sizes are kept small enough for the oracle to finish each case in well under
a second (m*n*k <= 6e7).
"""
import numpy as np
import pytest
import torch

import fp8_weight_only_amd as fw
import oracle
import workloads
from parity_util import assert_gate, assert_same_bits, oracle_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NAMES = {fw.PATH_GEMV: "gemv", fw.PATH_SKINNY: "skinny", fw.PATH_BATCH: "batch", fw.PATH_FALLBACK: "fallback"}
GUARD = 64  # guard elements / bytes around every buffer


def _draw(i):
    r = np.random.default_rng([20261202, i])
    kind = r.choice(["a256", "a16", "a8", "even", "odd"], p=[0.45, 0.15, 0.2, 0.12, 0.08])
    if kind == "a256":
        k = 256 * int(r.integers(1, 25))
    elif kind == "a16":
        k = 16 * int(r.integers(17, 400))
        k += 16 if k % 256 == 0 else 0
    elif kind == "a8":
        k = 8 * (2 * int(r.integers(16, 400)) + 1)
    elif kind == "even":
        k = 2 * int(r.integers(1, 3000))
        k += 2 if k % 8 == 0 else 0
    else:
        k = 2 * int(r.integers(0, 3000)) + 1
    band = r.choice(5, p=[0.25, 0.3, 0.15, 0.18, 0.12])
    m = [1, int(r.integers(2, 9)), int(r.integers(9, 17)), int(r.integers(17, 33)), int(r.integers(33, 101))][band]
    if r.random() < 0.15:
        n = int(r.choice([4096, 8192, 8200, 12288, 14336, 16400, 28672]))
    else:
        n = int(r.integers(1, 2049))
    n = max(1, min(n, int(6e7) // (m * k), int(3e7) // k))
    dtype = torch.bfloat16 if r.random() < 0.5 else torch.float16
    bias = bool(r.random() < 0.7)
    x_off = int(r.choice([0, 8, 4, 1], p=[0.75, 0.1, 0.05, 0.1]))          # elements
    q_off = int(r.choice([0, 16, 8, 4, 2, 1], p=[0.65, 0.1, 0.1, 0.1, 0.03, 0.02]))  # bytes
    y_off = int(r.choice([0, 1], p=[0.8, 0.2]))                               # elements
    empty_ws = bool(r.random() < 0.2)
    return (i, m, n, k, dtype, bias, x_off, q_off, y_off, empty_ws)


CASES = [_draw(i) for i in range(256)]


def _alignment(ptr):
    a = 1
    while a < 16 and ptr % (2 * a) == 0:
        a *= 2
    return a


def _expected_path(m, k, xa, qa):
    """The dispatch rule of fp8w_linear, written out from its documentation."""
    if m >= 1 and k >= 256 and k % 256 == 0 and xa >= 16 and qa >= 16:
        return fw.PATH_GEMV if m == 1 else fw.PATH_SKINNY if m <= 32 else fw.PATH_BATCH
    if m == 1 and k >= 256 and k % 8 == 0 and xa >= 16 and qa >= 8:
        return fw.PATH_GEMV
    if 1 <= m <= 32 and k >= 512 and k % 8 == 0 and xa >= 16 and qa >= 4:
        return fw.PATH_SKINNY
    return fw.PATH_FALLBACK


def _ids(c):
    i, m, n, k, dtype, bias, x_off, q_off, y_off, empty_ws = c
    return f"{i}-m{m}-n{n}-k{k}-{'bf16' if dtype == torch.bfloat16 else 'fp16'}-xo{x_off}-qo{q_off}-yo{y_off}" + \
        ("-nows" if empty_ws else "")


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_random_shape_parity(case):
    i, m, n, k, dtype, bias, x_off, q_off, y_off, empty_ws = case
    print(f"sweep {_ids(case)} bias={bias}", flush=True)
    c = workloads.random_case(5000 + i, m, n, k, dtype, with_bias=bias)
    q0, s = fw.quantize(torch.from_numpy(c.layer.w).to(DEV))
    b = None if c.layer.bias is None else c.layer.bias.to(DEV)

    xbuf = torch.zeros(x_off + m * k + GUARD, dtype=dtype, device=DEV)
    x = xbuf[x_off:x_off + m * k].view(m, k)
    x.copy_(c.x.to(DEV))
    qbuf = torch.zeros(q_off + n * k + GUARD, dtype=torch.uint8, device=DEV)
    q = qbuf[q_off:q_off + n * k].view(n, k)
    q.copy_(q0)
    ybuf = torch.full((y_off + m * n + GUARD,), float("nan"), dtype=dtype, device=DEV)
    y = ybuf[y_off:y_off + m * n].view(m, n)
    before = ybuf.clone()

    path = _expected_path(m, k, _alignment(x.data_ptr()), _alignment(q.data_ptr()))
    assert fw.linear_path(x, q) == path, f"dispatcher chose {NAMES[fw.linear_path(x, q)]}, rule says {NAMES[path]}"
    act = fw.BF16 if dtype == torch.bfloat16 else fw.FP16
    assert fw.fp8w_linear_kernel(fw.PATH_AUTO, m, n, k, act, x.data_ptr(), q.data_ptr())

    ws = torch.empty(0, dtype=torch.uint8, device=DEV) if empty_ws else None
    if empty_ws and path == fw.PATH_FALLBACK:
        with pytest.raises(RuntimeError):
            fw.linear(x, q, s, b, out=y, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ybuf.view(torch.int16), before.view(torch.int16)), "refused call wrote to y"
        return
    fw.linear(x, q, s, b, out=y, workspace=ws)
    torch.cuda.synchronize()

    yb = ybuf.view(torch.int16).cpu()
    bb = before.view(torch.int16).cpu()
    assert torch.equal(yb[:y_off], bb[:y_off]) and torch.equal(yb[y_off + m * n:], bb[y_off + m * n:]), \
        "write outside y"
    q_ref, s_ref, x64, y_ref, amax = oracle_case(c.layer.w, c.x, c.layer.bias)
    assert_same_bits(q.cpu().numpy(), q_ref, "codes (after the call)")
    assert_same_bits(s.cpu().numpy(), s_ref, "scales")
    assert torch.equal(x.cpu().view(torch.int16), c.x.view(torch.int16)), "x changed"
    assert_gate(y.double().cpu().numpy(), y_ref, x64, amax, f"sweep {_ids(case)} path={NAMES[path]}")


def _draw_grouped(i):
    r = np.random.default_rng([20261203, i])
    g = int(r.choice([32, 64, 128]))
    if r.random() < 0.55:
        k = 256 * int(r.integers(1, 25))
    else:
        k = g * int(r.integers(1, 6144 // g + 1))
    band = r.choice(5, p=[0.25, 0.3, 0.15, 0.18, 0.12])
    m = [1, int(r.integers(2, 9)), int(r.integers(9, 17)), int(r.integers(17, 33)), int(r.integers(33, 101))][band]
    n = int(r.choice([4096, 8192, 12288, 14336])) if r.random() < 0.15 else int(r.integers(1, 2049))
    n = max(1, min(n, int(6e7) // (m * k), int(3e7) // k))
    dtype = torch.bfloat16 if r.random() < 0.5 else torch.float16
    bias = bool(r.random() < 0.7)
    x_off = int(r.choice([0, 8, 1], p=[0.8, 0.1, 0.1]))           # elements
    q_off = int(r.choice([0, 16, 4], p=[0.8, 0.1, 0.1]))          # bytes
    empty_ws = bool(r.random() < 0.3)
    return (i, m, n, k, g, dtype, bias, x_off, q_off, empty_ws)


GROUPED = [_draw_grouped(i) for i in range(96)]


def _gids(c):
    i, m, n, k, g, dtype, bias, x_off, q_off, empty_ws = c
    return f"{i}-m{m}-n{n}-k{k}-g{g}-{'bf16' if dtype == torch.bfloat16 else 'fp16'}-xo{x_off}-qo{q_off}" + \
        ("-nows" if empty_ws else "")


@pytest.mark.parametrize("case", GROUPED, ids=[_gids(c) for c in GROUPED])
def test_random_grouped_parity(case):
    i, m, n, k, g, dtype, bias, x_off, q_off, empty_ws = case
    print(f"grouped sweep {_gids(case)} bias={bias}", flush=True)
    r = np.random.default_rng([7, i])
    w = r.standard_normal((n, k)).astype(np.float32)
    w *= (np.float32(10.0) ** r.uniform(-2, 1, (n, k // g)).astype(np.float32)).repeat(g, axis=1)
    c = workloads.random_case(7000 + i, m, n, k, dtype, with_bias=bias)
    q0, s = fw.quantize_grouped(torch.from_numpy(w).to(DEV), g)
    b = None if c.layer.bias is None else c.layer.bias.to(DEV)
    xbuf = torch.zeros(x_off + m * k + GUARD, dtype=dtype, device=DEV)
    x = xbuf[x_off:x_off + m * k].view(m, k)
    x.copy_(c.x.to(DEV))
    qbuf = torch.zeros(q_off + n * k + GUARD, dtype=torch.uint8, device=DEV)
    q = qbuf[q_off:q_off + n * k].view(n, k)
    q.copy_(q0)
    ybuf = torch.full((m * n + GUARD,), float("nan"), dtype=dtype, device=DEV)
    y = ybuf[:m * n].view(m, n)

    fast = k >= 256 and k % 256 == 0 and _alignment(x.data_ptr()) >= 16 and _alignment(q.data_ptr()) >= 16
    path = (fw.PATH_GEMV if m == 1 else fw.PATH_SKINNY if m <= 32 else fw.PATH_BATCH) if fast else fw.PATH_FALLBACK
    act = fw.BF16 if dtype == torch.bfloat16 else fw.FP16
    assert fw.fp8w_linear_grouped_path(m, n, k, g, act, x.data_ptr(), q.data_ptr()) == path
    assert fw.fp8w_linear_grouped_kernel(fw.PATH_AUTO, m, n, k, g, act, x.data_ptr(), q.data_ptr())
    ws = torch.empty(0, dtype=torch.uint8, device=DEV) if empty_ws else None
    fw.linear_grouped(x, q, s, b, out=y, workspace=ws)
    torch.cuda.synchronize()

    assert bool(torch.isnan(ybuf[m * n:].float()).all()), "write outside y"
    q_ref, s_ref, st = oracle.quantize_groups(w, g)
    assert st == 0
    assert_same_bits(q.cpu().numpy(), q_ref, "codes (after the call)")
    assert_same_bits(s.cpu().numpy(), s_ref, "scales")
    x64 = c.x.double().numpy()
    y_ref = oracle.linear_f64_groups(x64, q_ref, s_ref, g, None if c.layer.bias is None else c.layer.bias.double().numpy())
    assert_gate(y.double().cpu().numpy(), y_ref, x64, oracle.row_amax(w), f"grouped sweep {_gids(case)} path={NAMES[path]}")


def _draw_w8a8(i):
    r = np.random.default_rng([20261204, i])
    k = 256 * int(r.integers(1, 13))
    m = int(r.choice([int(r.integers(1, 33)), int(r.integers(33, 257)), int(r.integers(257, 700))], p=[0.3, 0.4, 0.3]))
    n = int(r.integers(1, 1500))
    n = max(1, min(n, int(6e7) // (m * k)))
    dtype = torch.bfloat16 if r.random() < 0.5 else torch.float16
    bias = bool(r.random() < 0.7)
    return (i, m, n, k, dtype, bias)


W8A8 = [_draw_w8a8(i) for i in range(64)]


def _wids(c):
    i, m, n, k, dtype, bias = c
    return f"{i}-m{m}-n{n}-k{k}-{'bf16' if dtype == torch.bfloat16 else 'fp16'}" + ("-bias" if bias else "")


@pytest.mark.parametrize("case", W8A8, ids=[_wids(c) for c in W8A8])
def test_random_w8a8_parity(case):
    """W8A8 ("Skill: Write an FP8 Kernel", "Required reasoning process" steps 2,
    4 and 5): the activation codes and scales bit for bit, every output within
    the gate against the oracle's fp64 layer on the same codes, nothing
    written outside y."""
    i, m, n, k, dtype, bias = case
    print(f"w8a8 sweep {_wids(case)}", flush=True)
    c = workloads.random_case(9000 + i, m, n, k, dtype, with_bias=bias)
    q, s = fw.quantize(torch.from_numpy(c.layer.w).to(DEV))
    x = c.x.to(DEV)
    qx, sx = fw.quantize_activations(x)
    qx_ref, sx_ref, st = oracle.quantize_activations(c.x.float().numpy())
    assert st == 0
    assert_same_bits(sx.cpu().numpy(), sx_ref, "activation scales")
    assert_same_bits(qx.cpu().numpy(), qx_ref, "activation codes")
    b = None if c.layer.bias is None else c.layer.bias.to(DEV)
    ybuf = torch.full((m * n + GUARD,), float("nan"), dtype=dtype, device=DEV)
    y = ybuf[:m * n].view(m, n)
    fw.linear_w8a8(x, q, s, b, out=y)
    torch.cuda.synchronize()
    assert bool(torch.isnan(ybuf[m * n:].float()).all()), "write outside y"
    q_ref, s_ref, _ = oracle.quantize_rows(c.layer.w)
    b64 = None if c.layer.bias is None else c.layer.bias.double().numpy()
    xd = oracle.decode(qx_ref) * sx_ref.astype(np.float64)[:, None]
    y_ref = oracle.linear_w8a8_f64(qx_ref, sx_ref, q_ref, s_ref, b64)
    assert_gate(y.double().cpu().numpy(), y_ref, xd, oracle.row_amax(c.layer.w), f"w8a8 sweep {_wids(case)}")
