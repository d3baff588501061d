"""Pins of the oracle's E4M3FNUZ decode and its carry-over to OCP codes.

Sources: "B04 - Precision & Quantization": the format table's "fp8
E4M3FNUZ" row (bias 8, maximum 240, minimum normal 7.8125e-3, minimum
subnormal 9.7656e-4, ulp(1) 0.125, 15 binades) and the footnote under it; the
section "Hardware support, and where the vendors diverge" (FNUZ: no
infinities, one NaN, no negative zero; the same bits decode a factor of two
apart from OCP); the trap list (0x80 is NaN in one format and -0.0 in the
other).
"""
import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
ALL = np.arange(256, dtype=np.uint8)


def test_printed_fnuz_row():
    with open(os.path.join(GOLDEN, "e4m3_format_row.json")) as f:
        row = json.load(f)["e4m3fnuz"]
    v = oracle.fnuz_decode(ALL)
    finite = v[np.isfinite(v)]
    pos = finite[finite > 0]
    rel = 1e-4
    assert math.isclose(finite.max(), row["max_finite"], rel_tol=rel)
    assert math.isclose(pos.min(), row["min_subnormal"], rel_tol=rel)
    assert math.isclose(oracle.fnuz_decode([0x08])[0], row["min_normal"], rel_tol=rel)
    one = int(np.flatnonzero(v == 1.0)[0])
    assert math.isclose(oracle.fnuz_decode([one + 1])[0] - 1.0, row["ulp1"], rel_tol=rel)
    exps = {math.frexp(x)[1] for x in pos if x >= row["min_normal"]}
    assert len(exps) == row["binades"]


def test_one_nan_no_negative_zero_no_infinity():
    v = oracle.fnuz_decode(ALL)
    assert list(np.flatnonzero(np.isnan(v))) == [0x80]
    assert np.all(np.isfinite(v[np.arange(256) != 0x80]))
    zeros = np.flatnonzero(v == 0.0)
    assert list(zeros) == [0x00] and math.copysign(1.0, v[0]) > 0
    assert v[0x7F] == 240.0 and v[0xFF] == -240.0


def test_same_bits_decode_a_factor_of_two_apart():
    """Every pattern both formats read as a finite non-zero number is worth
    exactly half in FNUZ; the exceptions are 0x80 (-0 vs NaN) and 0x7F/0xFF
    (NaN in OCP, +-240 in FNUZ)."""
    f, o = oracle.fnuz_decode(ALL), oracle.decode(ALL)
    both = np.isfinite(f) & np.isfinite(o) & (o != 0)
    assert both.sum() == 252
    assert np.array_equal(f[both], o[both] / 2)
    assert set(np.flatnonzero(~both)) == {0x00, 0x7F, 0x80, 0xFF}


def test_carry_over_keeps_values_but_the_sixteen_midpoints():
    """FNUZ values below 2^-6 with an odd mantissa fall exactly halfway
    between OCP subnormals (steps of 2^-9); they round to the even neighbour,
    2^-10 away. Every other finite code keeps its value exactly."""
    f = oracle.fnuz_decode(ALL)
    ocp = oracle.fnuz_to_ocp(ALL)
    back = oracle.decode(ocp)
    fin = np.isfinite(f)
    moved = np.flatnonzero(fin & (back != f))
    expect = [c for c in range(256) if c != 0x80 and (c >> 3) & 15 in (0, 1) and c & 1]
    assert sorted(moved) == expect and len(expect) == 16
    assert np.all(np.abs(back[moved] - f[moved]) == 2.0 ** -10)
    assert np.all((oracle.decode(ocp[moved]) / 2.0 ** -9) % 2 == 0)   # the even neighbour
    assert ocp[0x80] == 0x7F                                           # NaN stays NaN
    assert ocp[0x7F] == 0x77 and ocp[0xFF] == 0xF7                     # +-240 = 1.875 * 2^7


def test_carry_over_of_a_quantized_fnuz_row():
    """A row quantized the FNUZ way (scale = amax / 240, codes of w / scale)
    carries over with its scale unchanged: value_ocp(new code) * scale is the
    FNUZ reconstruction, up to the 2^-10 midpoint moves."""
    rng = np.random.default_rng(0)
    w = rng.standard_normal(4096)
    s = np.abs(w).max() / 240.0
    fin = oracle.fnuz_decode(ALL)
    order = np.argsort(fin[np.isfinite(fin)])
    vals = fin[np.isfinite(fin)][order]
    codes_f = np.flatnonzero(np.isfinite(fin))[order]
    idx = np.abs(vals[None, :] - (w / s)[:, None]).argmin(axis=1)  # nearest FNUZ code (ties: either)
    q_fnuz = codes_f[idx].astype(np.uint8)
    recon_fnuz = fin[q_fnuz] * s
    recon_ocp = oracle.decode(oracle.fnuz_to_ocp(q_fnuz)) * s
    assert np.all(np.abs(recon_ocp - recon_fnuz) <= 2.0 ** -10 * s)
