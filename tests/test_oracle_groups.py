"""Pins of the oracle's group-wise scales along k.

Sources: "B04 - Precision & Quantization", sections "Post-training quantization
versus quantization-aware training" (one scale per run of g = 32 / 64 / 128
weights of a row) and "The one that matters: quantization is a quality
decision" (per-channel -> per-group); the Day-98 lab page's storage census
("one scale per 32": the block's max |w| / 448, the cast of w / scale); "FP8
weight-only (precision: fp8_weights)", section "The contract" for what each
group then does (amax / 448, round to nearest even, clamp to +-448).

The pins do not re-type the formulas: each group must be quantized exactly as
the (separately pinned) row quantizer quantizes that group on its own; g = k
must reduce to the per-channel oracle; closed forms, one-hot columns and exact
rational arithmetic fix the linear layer's group indexing.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GROUPS = (32, 64, 128)


def _qg(w, g):
    q, s, st = oracle.quantize_groups(w, g)
    assert st == 0
    return q, s


@pytest.mark.parametrize("g", GROUPS)
def test_each_group_is_quantized_as_its_own_row(g):
    """Group j of row n has the scale and codes the row quantizer gives the
    slice W[n, j*g:(j+1)*g] on its own: a scale indexed by the wrong group, or an
    amax taken across groups, fails here."""
    rng = np.random.default_rng(g)
    n, k = 24, 8 * g
    w = (rng.standard_normal((n, k)) * rng.uniform(1e-3, 1e3, (n, k // g)).repeat(g, axis=1)).astype(np.float32)
    w[5, 2 * g:3 * g] = 0.0  # a zero group
    q, s = _qg(w, g)
    assert s.shape == (n, k // g)
    for j in range(k // g):
        qj, sj, st = oracle.quantize_rows(np.ascontiguousarray(w[:, j * g:(j + 1) * g]))
        assert st == 0
        assert np.array_equal(s[:, j].view(np.uint32), sj.view(np.uint32)), j
        assert np.array_equal(q[:, j * g:(j + 1) * g], qj), j
    assert s[5, 2] == 0.0 and np.all(q[5, 2 * g:3 * g] == 0)


def test_group_of_the_whole_row_is_per_channel():
    w = workloads.random_case(8, 1, 40, 256, torch.bfloat16).layer.w
    q, s = _qg(w, 256)
    q1, s1, _ = oracle.quantize_rows(w)
    assert np.array_equal(q, q1) and np.array_equal(s[:, 0].view(np.uint32), s1.view(np.uint32))


def test_anchored_groups_give_power_of_two_scales_and_golden_codes():
    """Group 0 is anchored at 448 and group 1 at 896: their scales are exactly 1
    and 2, so group 0's codes are the hand-derived round-to-nearest-even cases and
    group 1 (twice the same inputs) the same codes."""
    with open(os.path.join(GOLDEN, "rne_cases.json")) as f:
        cases = [c for c in json.load(f)["cases"] if c["t"] != "inf"]
    vals = [float.fromhex(c["t"]) for c in cases if abs(float.fromhex(c["t"])) <= 448.0][:31]
    codes = [c["code"] for c in cases if abs(float.fromhex(c["t"])) <= 448.0][:31]
    vals += [0.0] * (31 - len(vals))
    codes += [0] * (31 - len(codes))
    g0 = [448.0] + vals
    g1 = [896.0] + [2.0 * v for v in vals]
    w = np.array([g0 + g1], dtype=np.float32)
    q, s = _qg(w, 32)
    assert s[0, 0] == np.float32(1.0) and s[0, 1] == np.float32(2.0)
    assert q[0, 0] == 0x7E and q[0, 32] == 0x7E
    assert list(q[0, 1:32]) == codes and list(q[0, 33:64]) == codes


@pytest.mark.parametrize("g", GROUPS)
def test_group_amax_encodes_to_448(g):
    rng = np.random.default_rng(3 * g)
    n, k = 64, 4 * g
    w = (rng.standard_normal((n, k)) * rng.uniform(1e-20, 1e20, (n, k)).astype(np.float64) ** 0.1).astype(np.float32)
    q, s = _qg(w, g)
    for j in range(k // g):
        blk = w[:, j * g:(j + 1) * g]
        arg = np.abs(blk).argmax(axis=1)
        got = q[np.arange(n), j * g + arg]
        neg = blk[np.arange(n), arg] < 0
        assert np.all(np.where(neg, got == 0xFE, got == 0x7E))


def test_nonfinite_weight_is_rejected():
    w = np.ones((2, 64), dtype=np.float32)
    w[1, 40] = np.inf
    _, _, st = oracle.quantize_groups(w, 32)
    assert st == 3


def test_group_scales_shrink_the_error_of_an_outlier_row():
    """The reason for the finer granularity ([B04]): one outlier inside a row
    coarsens only its own group. e4m3 keeps its relative precision until values
    fall into the subnormal binade (below 2^-6 of the scale unit), so the
    outlier here is 1e5x: per channel it pushes the row's typical weights
    down to ~1e-3 in code units, subnormal; per group only group 0 suffers."""
    rng = np.random.default_rng(4)
    w = rng.standard_normal((8, 512)).astype(np.float32)
    w[:, 7] = 1e5
    q1, s1, _ = oracle.quantize_rows(w)
    qg, sg = _qg(w, 32)
    per_channel = oracle.weight_error(w, q1, s1)
    per_group = oracle.weight_error_groups(w, qg, sg, 32)
    assert per_group["rel_l2"] < per_channel["rel_l2"]
    assert per_group["underflow"] < per_channel["underflow"]
    rest = np.s_[:, 32:]
    err_g = oracle.dequantize_groups_f64(qg, sg, 32)[rest] - w[rest]
    err_c = oracle.dequantize_f64(q1, s1)[rest] - w[rest]
    ref = np.linalg.norm(w[rest])
    assert np.linalg.norm(err_g) < 0.035 * ref   # the Gaussian level, ~2.6 %
    assert np.linalg.norm(err_c) > 0.10 * ref    # subnormal codes per channel


@pytest.mark.parametrize("g", GROUPS)
def test_linear_all_ones_closed_form(g):
    """x = 1 and W[n, group j] = c[n, j]: every code is 0x7E, so
    y[m, n] = sum_j fl32(c[n, j] / 448) * 448 * g + b[n]."""
    ng = 5
    c = np.array([[0.02, 1.0, 3.3e-3, 123.0, 7.0], [5.0, 1e-3, 2.5, 0.75, 11.0]], dtype=np.float32)
    w = np.repeat(c, g, axis=1)
    q, s = _qg(w, g)
    assert np.all(q == 0x7E)
    x = np.ones((3, ng * g))
    b = np.array([0.5, -1.0])
    y = oracle.linear_f64_groups(x, q, s, g, b)
    expect = ((c / np.float32(448.0)).astype(np.float64) * 448.0 * g).sum(axis=1) + b
    assert np.allclose(y, np.broadcast_to(expect, (3, 2)), rtol=1e-15, atol=0)


@pytest.mark.parametrize("g", GROUPS)
def test_linear_one_hot_picks_the_columns_group_scale(g):
    rng = np.random.default_rng(5 + g)
    n, k = 19, 4 * g
    w = (rng.standard_normal((n, k)) * rng.uniform(1e-2, 1e2, (n, k // g)).repeat(g, axis=1)).astype(np.float32)
    q, s = _qg(w, g)
    b = rng.standard_normal(n)
    table = oracle.decode(np.arange(256))
    for j in (0, 1, g - 1, g, 2 * g + 5, k - 1):
        x = np.zeros((1, k))
        x[0, j] = 1.0
        y = oracle.linear_f64_groups(x, q, s, g, b)[0]
        assert np.array_equal(y, s[:, j // g].astype(np.float64) * table[q[:, j]] + b), j
        assert np.array_equal(y, oracle.dequantize_groups_f64(q, s, g)[:, j] + b), j


def test_linear_tiny_exact_rational_brute_force():
    """M=2, N=3, K=64, g=32 with random codes and scales: exact rational
    arithmetic agrees with the fp64 oracle to within a few fp64 roundings."""
    rng = np.random.default_rng(6)
    g, k = 32, 64
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    q = rng.choice(finite, size=(3, k)).astype(np.uint8)
    s = rng.uniform(1e-4, 1e-1, (3, k // g)).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((2, k)).astype(np.float32)).to(torch.bfloat16).double().numpy()
    b = rng.standard_normal(3)
    y = oracle.linear_f64_groups(x, q, s, g, b)
    vals = oracle.decode(np.arange(256))
    for m in range(2):
        for n in range(3):
            exact = Fraction(float(b[n]))
            for j in range(k // g):
                part = sum(Fraction(float(x[m, i])) * Fraction(float(vals[q[n, i]])) for i in range(j * g, (j + 1) * g))
                exact += Fraction(float(s[n, j])) * part
            scale_of_terms = sum(abs(Fraction(float(s[n, i // g])) * Fraction(float(x[m, i])) *
                                     Fraction(float(vals[q[n, i]]))) for i in range(k)) + abs(Fraction(float(b[n])))
            assert abs(Fraction(float(y[m, n])) - exact) <= scale_of_terms * Fraction(2) ** -48


def test_linear_equal_group_scales_reduce_to_per_channel():
    c = workloads.random_case(9, 3, 30, 256, torch.bfloat16)
    q, s, _ = oracle.quantize_rows(c.layer.w)
    x = c.x.double().numpy()
    b = c.layer.bias.double().numpy()
    sg = np.repeat(s[:, None], 256 // 32, axis=1)
    y_g = oracle.linear_f64_groups(x, q, sg, 32, b)
    y_c = oracle.linear_f64(x, q, s, b)
    assert np.allclose(y_g, y_c, rtol=1e-13, atol=1e-13)


def test_linear_matches_dequantized_weight_matmul():
    c = workloads.random_case(10, 5, 70, 256, torch.float16)
    q, s = _qg(c.layer.w, 64)
    x = c.x.double().numpy()
    b = c.layer.bias.double().numpy()
    y = oracle.linear_f64_groups(x, q, s, 64, b)
    assert np.allclose(y, x @ oracle.dequantize_groups_f64(q, s, 64).T + b, rtol=1e-12, atol=1e-12)
    rows = np.array([0, 4, 2])
    cols = np.array([69, 0, 33])
    assert np.array_equal(oracle.linear_f64_groups_sampled(x, q, s, 64, b, rows, cols), y[rows, cols])


def test_weight_error_groups_reduces_to_per_channel():
    w = workloads.random_case(11, 1, 20, 128, torch.bfloat16).layer.w
    q, s, _ = oracle.quantize_rows(w)
    a = oracle.weight_error(w, q, s)
    b = oracle.weight_error_groups(w, q, s[:, None], 128)
    # the totals are OpenMP reductions, whose order may differ between calls
    assert abs(a["rel_l2"] - b["rel_l2"]) <= 1e-12 * a["rel_l2"]
    for key in ("worst_channel_rel_l2", "underflow", "crest_max", "crest_median"):
        assert a[key] == b[key], key
