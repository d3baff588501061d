"""Pins of the oracle's fp64 linear layer and output metrics.

Sources: "FP8 weight-only (precision: fp8_weights)", section "The contract"
(y[m,n] = scale[n] * sum_k x[m,k] q[n,k] + bias[n]; "Fallback": the dequantised
weight q.float() * scale[:, None] gives the same numerics); "Inference with
NVFP4/MXFP8" (cuTile-rs), sections on the runnable examples: the all-ones input
check; "Skill: Write an FP8 Kernel", step 7: scale = 0 (all-zero weights).
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
import workloads


def _q(w):
    q, s, st = oracle.quantize_rows(w)
    assert st == 0
    return q, s


def test_all_ones_closed_form():
    """x = 1 everywhere and rows W[n,:] = c_n: every code is 0x7E (448), so
    y[m,n] = fl32(c_n / 448) * 448 * K + b[n]."""
    K = 1000
    c = np.array([0.02, 1.0, 3.3e-3, 123.0, 7.0], dtype=np.float32)
    w = np.repeat(c[:, None], K, axis=1)
    q, s = _q(w)
    assert np.all(q == 0x7E)
    x = np.ones((3, K))
    b = np.array([0.5, -1.0, 0.0, 2.0, 0.25])
    y = oracle.linear_f64(x, q, s, b)
    expect = (c / np.float32(448.0)).astype(np.float64) * 448.0 * K + b
    assert np.array_equal(y, np.broadcast_to(expect, (3, 5)))


def test_one_hot_selects_a_column():
    """x = e_j picks y[n] = scale[n] * value(q[n, j]) + bias[n]; a transposed
    weight or a shifted index would pick another element."""
    g = np.random.default_rng(1)
    n, k = 37, 53
    w = g.standard_normal((n, k)).astype(np.float32)
    q, s = _q(w)
    b = g.standard_normal(n)
    table = oracle.decode(np.arange(256))
    for j in (0, 1, 17, k - 1):
        x = np.zeros((1, k))
        x[0, j] = 1.0
        y = oracle.linear_f64(x, q, s, b)[0]
        assert np.array_equal(y, s.astype(np.float64) * table[q[:, j]] + b)


def test_zero_rows_give_bias_exactly():
    lay = workloads.block_layer(0)
    w = lay.w[:256].copy()
    w[3] = 0.0
    w[100] = 0.0
    q, s = _q(w)
    x = workloads.activations(9, 0, 4, w.shape[1], torch.bfloat16).double().numpy()
    b = np.linspace(-1, 1, 256)
    y = oracle.linear_f64(x, q, s, b)
    assert s[3] == 0.0 and s[100] == 0.0
    assert np.all(y[:, 3] == b[3]) and np.all(y[:, 100] == b[100])


def test_tiny_exact_rational_brute_force():
    """M=2, N=3, K=8 with random codes and scales: exact rational arithmetic agrees
    with the fp64 oracle to within one fp64 rounding of the result."""
    g = np.random.default_rng(2)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    q = g.choice(finite, size=(3, 8)).astype(np.uint8)
    s = g.uniform(1e-4, 1e-1, 3).astype(np.float32)
    x = torch.from_numpy(g.standard_normal((2, 8)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    b = g.standard_normal(3)
    y = oracle.linear_f64(x, q, s, b)
    vals = oracle.decode(np.arange(256))
    for m in range(2):
        for n in range(3):
            acc = sum(Fraction(float(x[m, k])) * Fraction(float(vals[q[n, k]])) for k in range(8))
            exact = Fraction(float(s[n])) * acc + Fraction(float(b[n]))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(2) ** -50 + Fraction(2) ** -1060


def test_matches_dequantized_weight_matmul():
    """The fallback reading of the contract: x @ (value(q) * scale[:, None])^T + b,
    here through numpy's float64 matmul, gives the same layer."""
    c = workloads.random_case(3, 5, 70, 130, torch.bfloat16)
    q, s = _q(c.layer.w)
    x = c.x.double().numpy()
    b = c.layer.bias.double().numpy()
    y = oracle.linear_f64(x, q, s, b)
    ref = x @ oracle.dequantize_f64(q, s).T + b
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_sampled_equals_full():
    c = workloads.random_case(4, 6, 40, 96, torch.float16)
    q, s = _q(c.layer.w)
    x = c.x.double().numpy()
    b = c.layer.bias.double().numpy()
    y = oracle.linear_f64(x, q, s, b)
    rows = np.array([0, 5, 3, 2])
    cols = np.array([39, 0, 17, 17])
    assert np.array_equal(oracle.linear_f64_sampled(x, q, s, b, rows, cols), y[rows, cols])


def test_quantized_layer_tracks_original_weight():
    """Output-level quality of the method on a Gaussian layer: cosine to the
    unquantized layer stays near 1 (the "near-lossless" report)."""
    c = workloads.random_case(5, 4, 512, 1024, torch.bfloat16)
    q, s = _q(c.layer.w)
    x = c.x.double().numpy()
    b = c.layer.bias.double().numpy()
    y = oracle.linear_f64(x, q, s, b)
    y_orig = x @ c.layer.w.astype(np.float64).T + b
    met = oracle.output_metrics(y, y_orig)
    assert met["min_cosine"] > 0.999
    assert met["max_rel_l2"] < 0.05


def test_output_metrics_closed_forms():
    y = np.array([[1.0, 2.0, 2.0], [0.0, 3.0, 4.0]])
    m = oracle.output_metrics(y, y)
    assert m["min_cosine"] == 1.0 and m["max_rel_l2"] == 0.0
    m2 = oracle.output_metrics(2 * y, y)
    assert abs(m2["min_cosine"] - 1.0) < 1e-15 and abs(m2["max_rel_l2"] - 1.0) < 1e-15
    m3 = oracle.output_metrics(-y, y)
    assert abs(m3["min_cosine"] + 1.0) < 1e-15 and abs(m3["max_rel_l2"] - 2.0) < 1e-15
