"""Pins of the oracle's build-time quantizer and weight-error report.

Sources: "FP8 weight-only (precision: fp8_weights)", section "The contract"
(scale = amax(|row|)/448 per output channel, codes round(w/scale) to nearest
even clamped to +-448, error report rel_l2 / worst_channel_rel_l2 / underflow /
crest); "Skill: Write an FP8 Kernel", "Required reasoning process" step 2
(amax -> scale -> cast(x/scale)) and step 7 (scale = 0 without a division).
"""
import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_anchor_row_gives_unit_scale_and_golden_codes():
    """A row whose amax is 448 has scale exactly 1, so its codes are the encoder's
    hand-derived round-to-nearest-even cases taken through the quantizer."""
    with open(os.path.join(GOLDEN, "rne_cases.json")) as f:
        cases = [c for c in json.load(f)["cases"] if c["t"] != "inf"]
    vals = [float.fromhex(c["t"]) for c in cases]
    vals = [v for v in vals if abs(v) <= 448.0]
    codes = [c["code"] for c in cases if abs(float.fromhex(c["t"])) <= 448.0]
    w = np.array([[448.0] + vals], dtype=np.float32)
    q, scale, st = oracle.quantize_rows(w)
    assert st == 0
    assert scale[0] == np.float32(1.0)
    assert q[0, 0] == 0x7E
    assert list(q[0, 1:]) == codes


def test_scale_is_fp32_quotient_of_amax():
    w = np.array([[1.0, -0.5], [-3.0, 2.0], [0.0, 7e-3]], dtype=np.float32)
    q, scale, st = oracle.quantize_rows(w)
    assert st == 0
    # fl32(amax / 448) for amax = 1, 3, 7e-3 (numpy float32 division is IEEE)
    assert scale[0] == np.float32(1.0) / np.float32(448.0)
    assert scale[1] == np.float32(3.0) / np.float32(448.0)
    assert scale[2] == np.float32(7e-3) / np.float32(448.0)


def test_amax_element_encodes_to_448_on_every_row():
    g = np.random.default_rng(11)
    n, k = 512, 300
    w = (g.standard_normal((n, k)) * g.uniform(1e-30, 1e30, (n, 1))).astype(np.float32)
    q, scale, st = oracle.quantize_rows(w)
    assert st == 0
    arg = np.abs(w).argmax(axis=1)
    sgn = w[np.arange(n), arg] < 0
    got = q[np.arange(n), arg]
    assert np.all(np.where(sgn, got == 0xFE, got == 0x7E))
    # every code's magnitude stays within the finite range
    assert not np.any((q & 0x7F) == 0x7F)


def test_quantization_error_bound():
    """|value(q) * scale - w| is at most half an e4m3 step of w/scale (plus the fp32
    rounding of the quotient), and never above 2^-4 * |w| for normals or 2^-10 * scale
    in the subnormal binade."""
    g = np.random.default_rng(5)
    w = (g.standard_t(3.0, size=(64, 4096)) * 0.02).astype(np.float32)
    q, scale, _ = oracle.quantize_rows(w)
    deq = oracle.dequantize_f64(q, scale)
    t = np.abs(w.astype(np.float64) / scale[:, None].astype(np.float64))
    err = np.abs(deq - w.astype(np.float64)) / scale[:, None]
    normal = t >= 2.0 ** -6
    step = np.where(normal, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(err <= 0.5 * step * (1 + 2 ** -20) + t * 2 ** -23)


def test_zero_row_scale_zero_codes_zero():
    w = np.zeros((3, 17), dtype=np.float32)
    w[1, 4] = -2.5
    q, scale, st = oracle.quantize_rows(w)
    assert st == 0
    assert scale[0] == 0.0 and scale[2] == 0.0
    assert not q[0].any() and not q[2].any()
    # signed zeros in an all-zero row are plain 0x00 (no division happens)
    wz = np.array([[-0.0, 0.0, -0.0]], dtype=np.float32)
    qz, sz, _ = oracle.quantize_rows(wz)
    assert sz[0] == 0.0 and list(qz[0]) == [0, 0, 0]


def test_nonfinite_weights_rejected():
    for bad in (np.nan, np.inf, -np.inf):
        w = np.ones((2, 8), dtype=np.float32)
        w[1, 3] = bad
        _, _, st = oracle.quantize_rows(w)
        assert st == 3


def test_negative_underflow_is_minus_zero():
    w = np.array([[448.0, -2.0 ** -11, 2.0 ** -11, -1e-30]], dtype=np.float32)
    q, _, _ = oracle.quantize_rows(w)
    assert list(q[0]) == [0x7E, 0x80, 0x00, 0x80]


def test_weight_error_closed_forms():
    # row 0: [448, 1.0625] -> scale 1, codes [0x7E, 0x38] -> What = [448, 1]
    # row 1: [448, 2^-11] -> the small weight underflows to 0
    # row 2: zero row
    w = np.array([[448.0, 1.0625], [448.0, 2.0 ** -11], [0.0, 0.0]], dtype=np.float32)
    q, scale, _ = oracle.quantize_rows(w)
    rep = oracle.weight_error(w, q, scale)
    n0 = math.hypot(448.0, 1.0625)
    ch0 = 0.0625 / n0
    ch1 = 2.0 ** -11 / math.hypot(448.0, 2.0 ** -11)
    assert rep["channel_rel_l2"][0] == ch0
    assert abs(rep["channel_rel_l2"][1] - ch1) <= 1e-15
    assert rep["channel_rel_l2"][2] == 0.0
    assert rep["worst_channel_rel_l2"] == max(ch0, ch1)
    tot = math.sqrt(0.0625 ** 2 + 2.0 ** -22) / math.sqrt(448.0 ** 2 * 2 + 1.0625 ** 2 + 2.0 ** -22)
    assert abs(rep["rel_l2"] - tot) <= 1e-15
    assert rep["underflow"] == 1 / 4
    crest0 = 448.0 / math.sqrt((448.0 ** 2 + 1.0625 ** 2) / 2)
    crest1 = 448.0 / math.sqrt((448.0 ** 2 + 2.0 ** -22) / 2)
    assert abs(rep["crest_max"] - max(crest0, crest1)) <= 1e-12


def test_gaussian_rows_error_is_a_few_percent():
    """Sanity (derived, not printed by the pages): 3 mantissa bits give a relative
    rounding error of about 2-3 % on Gaussian rows and almost no underflow."""
    g = np.random.default_rng(9)
    w = (g.standard_normal((256, 2048)) * 0.02).astype(np.float32)
    q, scale, _ = oracle.quantize_rows(w)
    rep = oracle.weight_error(w, q, scale)
    assert 0.015 < rep["rel_l2"] < 0.035
    assert rep["underflow"] < 1e-3


def test_row_amax_hand_rows():
    """max_k |W[n,k]| per output row ("The contract": the scale's amax is taken over
    one output channel's row). Hand-written rows whose answers are read off by eye:
    the extreme is negative in one row, a row is all zeros (signed zeros included),
    one row holds a 50x outlier, and the matrix is not square, so a transposed
    index (max over a column) or a dropped absolute value gives a different answer."""
    w = np.array([[0.25, -3.5, 1.0, 2.0, -0.5],
                  [0.0, -0.0, 0.0, -0.0, 0.0],
                  [0.02, -0.01, 0.015, 1.0, -0.03],
                  [-1e-30, 2e-30, -4e-30, 0.0, 3e-30]], dtype=np.float32)
    got = oracle.row_amax(w)
    assert got.shape == (4,)
    assert got[0] == 3.5
    assert got[1] == 0.0 and not np.signbit(got[1])
    assert got[2] == 1.0
    assert got[3] == float(np.float32(4e-30))
    # the column maxima (what a transposed index would return) differ
    assert not np.array_equal(got[:4], np.abs(w).max(axis=0)[:4])
    # one element per row: |w|
    single = np.array([[-7.0], [0.125], [-0.0]], dtype=np.float32)
    assert list(oracle.row_amax(single)) == [7.0, 0.125, 0.0]


def test_row_amax_matches_numpy_on_outlier_rows():
    """Against numpy's own reduction on rows shaped like the decoder-block workload:
    Gaussian rows, some scaled 50x, some all zero, and rows whose extreme is negative."""
    g = np.random.default_rng(21)
    w = (g.standard_normal((300, 1000)) * 0.02).astype(np.float32)
    w[::17] *= 50.0
    w[5::29] = 0.0
    w[7, 11] = -abs(w[7]).max() * 3.0
    ref = np.abs(w.astype(np.float64)).max(axis=1)
    assert np.array_equal(oracle.row_amax(w), ref)


def test_row_amax_is_448_scale_within_one_ulp():
    """scale = fl32(amax / 448) is correctly rounded, so 448 * scale lies within one
    fp32 ulp of amax for every row with a normal scale, and amax is 0 exactly when
    the scale is 0."""
    g = np.random.default_rng(23)
    w = (g.standard_normal((400, 700)) * g.uniform(1e-20, 1e20, (400, 1))).astype(np.float32)
    w[3] = 0.0
    _, scale, st = oracle.quantize_rows(w)
    assert st == 0
    amax = oracle.row_amax(w)
    assert (amax == 0.0).tolist() == (scale == 0.0).tolist()
    nz = scale != 0
    ulp = np.spacing(amax[nz].astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(448.0 * scale[nz].astype(np.float64) - amax[nz]) <= ulp)
