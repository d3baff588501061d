"""Pins of the oracle's e4m3fn codec against what the pages fix.

Sources: "B04 - Precision & Quantization", section "The numbers, derived rather
than tabulated" (table row, footnote) and section "Hardware support, and where
the vendors diverge" (OCP vs FNUZ, 0x80 is -0 in OCP); "FP8 weight-only
(precision: fp8_weights)", sections "The contract" (round to nearest even,
clamp to +-448) and "Dequantise in registers" (every e4m3 value is a bf16
value).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FINITE = [c for c in range(256) if c not in (0x7F, 0xFF)]


def _row():
    with open(os.path.join(GOLDEN, "e4m3_format_row.json")) as f:
        return json.load(f)


def test_printed_table_row_matches_decode():
    row = _row()
    e4 = row["e4m3"]
    rel = row["printed_relative_precision"]
    vals = oracle.decode(FINITE)
    pos = vals[vals > 0]
    assert pos.max() == e4["max_finite"] == 448.0
    assert oracle.decode([0x7E])[0] == 448.0
    # smallest normal: first code of biased exponent 1
    assert oracle.decode([0x08])[0] == pytest.approx(e4["min_normal"], rel=rel)
    assert oracle.decode([0x08])[0] == 2.0 ** -6
    # smallest subnormal (printed 1.9531e-3, exact 2^-9)
    assert pos.min() == pytest.approx(e4["min_subnormal"], rel=rel)
    assert pos.min() == 2.0 ** -9
    # ulp(1): spacing just above 1.0
    assert oracle.decode([0x38])[0] == 1.0
    assert oracle.decode([0x39])[0] - 1.0 == e4["ulp1"]
    # binades of normal numbers: exponents -6 .. 8
    normals = pos[pos >= e4["min_normal"]]
    assert len({math.frexp(v)[1] for v in normals}) == e4["binades"]


def test_decode_is_not_fnuz():
    """The FNUZ row (bias 8, max 240) decodes the same bits a factor of two lower;
    the OCP format has 0x80 = -0.0 where FNUZ has its NaN."""
    fnuz = _row()["e4m3fnuz"]
    assert oracle.decode([0x7E])[0] == 2 * 224.0  # FNUZ 0x7E would be 224
    assert oracle.decode([0x7F])[0] != fnuz["max_finite"]
    z = oracle.decode([0x80])[0]
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


def test_nan_patterns_only_at_top():
    vals = oracle.decode(np.arange(256))
    nan_codes = [c for c in range(256) if np.isnan(vals[c])]
    assert nan_codes == [0x7F, 0xFF]
    assert not np.isinf(vals).any()


def test_decode_monotone_and_symmetric():
    pos = oracle.decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)
    neg = oracle.decode(np.arange(0x80, 0xFF))
    assert np.array_equal(neg, -pos)


def test_closed_form_binades():
    """Within a binade of exponent e the 8 values are (1 + m/8) 2^e, m = 0..7."""
    for be in range(1, 16):
        for m in range(8):
            c = (be << 3) | m
            if c == 0x7F:
                continue
            assert oracle.decode([c])[0] == (1 + m / 8) * 2.0 ** (be - 7)
    for m in range(8):
        assert oracle.decode([m])[0] == m * 2.0 ** -9


def test_round_trip_all_finite_codes():
    vals = oracle.decode(FINITE).astype(np.float32)
    codes = oracle.encode(vals)
    assert list(codes) == FINITE


def test_hand_derived_rne_cases():
    with open(os.path.join(GOLDEN, "rne_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        t = float("inf") if c["t"] == "inf" else float.fromhex(c["t"])
        assert oracle.encode_one(t) == c["code"], c
        assert oracle.encode_search_one(t) == c["code"], c


def test_nearest_code_brute_force():
    """For random fp32 inputs, no finite code is strictly nearer than the chosen one,
    and an exact tie picks the even code (linear scan over all 254 finite codes)."""
    g = np.random.default_rng(7)
    pos = oracle.decode(np.arange(0x7F))
    mids = 0.5 * (pos[1:] + pos[:-1])            # every tie, exact in fp32
    t = np.concatenate([
        g.uniform(-460, 460, 3000), g.uniform(-0.02, 0.02, 3000),
        g.standard_normal(3000) * 4, mids, -mids,
    ]).astype(np.float32)
    assert np.array_equal(t[-2 * len(mids):-len(mids)].astype(np.float64), mids)
    codes = oracle.encode(t)
    table = oracle.decode(FINITE)
    for ti, ci in zip(t.astype(np.float64), codes):
        target = min(max(ti, -448.0), 448.0)
        d = np.abs(table - target)
        best = d.min()
        cands = [FINITE[i] for i in np.flatnonzero(d == best)]
        if len(cands) > 1:
            cands = [c for c in cands if c % 2 == 0] or cands
            # +-0 tie: the sign follows the input
            if set(cands) == {0x00, 0x80}:
                cands = [0x80 if math.copysign(1.0, ti) < 0 else 0x00]
        assert ci in cands, (ti, hex(ci), [hex(c) for c in cands])


def test_two_encoders_agree_on_all_fp32_patterns():
    """Exhaustive: both independent encoders agree on every non-NaN fp32 bit pattern."""
    bad, first_bad = oracle.encoders_compare(0, 1 << 32)
    assert bad == 0, hex(first_bad)


def test_every_e4m3_value_is_exact_in_bf16_and_fp16():
    vals = oracle.decode(FINITE)
    assert np.array_equal(oracle.round_to_bf16(vals), vals)
    assert np.array_equal(oracle.round_to_f16(vals), vals)


def test_bf16_rounding_matches_library_cast():
    """The oracle's fp32 -> bf16 rounding equals torch's round-to-nearest-even cast,
    including exact ties (low half 0x8000) and values next to them."""
    g = np.random.default_rng(3)
    u = g.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    allu = np.concatenate([u, ties, ties + np.uint32(1), ties - np.uint32(1)])
    f = allu.view(np.float32)
    f = f[np.isfinite(f)]
    mine = oracle.round_bf16_bits(f)
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    # hand-derived ties: 1 + 2^-8 -> 1.0 (even) ; 1 + 3*2^-8 -> 1 + 2^-6 (even)
    assert oracle.round_to_bf16([1 + 2 ** -8])[0] == 1.0
    assert oracle.round_to_bf16([1 + 3 * 2 ** -8])[0] == 1 + 2 ** -6


def test_f16_rounding_matches_library_cast():
    """The oracle's value -> fp32 -> fp16 rounding equals torch's round-to-nearest-even
    cast on random fp32 patterns, on exact fp16 ties (the 13 dropped bits equal to
    0x1000) and their neighbours, in the subnormal range and at overflow."""
    g = np.random.default_rng(4)
    u = g.integers(0, 1 << 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # patterns inside fp16's normal range whose low 13 bits are a tie
    e = g.integers(113, 142, size=50000, dtype=np.uint64).astype(np.uint32)  # fp32 exponents 2^-14 .. 2^14
    s = g.integers(0, 2, size=50000, dtype=np.uint64).astype(np.uint32) << np.uint32(31)
    mant = g.integers(0, 1 << 10, size=50000, dtype=np.uint64).astype(np.uint32) << np.uint32(13)
    ties = s | (e << np.uint32(23)) | mant | np.uint32(0x1000)
    allu = np.concatenate([u, ties, ties + np.uint32(1), ties - np.uint32(1)])
    f = allu.view(np.float32)
    f = f[np.isfinite(f)]
    f = np.concatenate([f, (g.standard_normal(20000) * 2.0 ** -20).astype(np.float32),
                        np.array([65504.0, 65519.0, 65520.0, -65520.0, 7e4], dtype=np.float32)])
    mine = oracle.round_to_f16(f)
    ref = torch.from_numpy(f.copy()).to(torch.float16).double().numpy()
    assert np.array_equal(mine, ref, equal_nan=True)
    # hand-derived ties: 1 + 2^-11 -> 1.0 (even); 1 + 3*2^-11 -> 1 + 2^-9 (even);
    # 2^-25 (half the smallest subnormal) -> +0; 3*2^-25 -> 2^-23 (even);
    # 65520 (halfway between 65504 and 2^16) -> inf; 65519 -> 65504
    assert oracle.round_to_f16([1 + 2 ** -11])[0] == 1.0
    assert oracle.round_to_f16([1 + 3 * 2 ** -11])[0] == 1 + 2 ** -9
    assert oracle.round_to_f16([2.0 ** -25])[0] == 0.0
    assert oracle.round_to_f16([3 * 2.0 ** -25])[0] == 2.0 ** -23
    assert oracle.round_to_f16([65520.0])[0] == np.inf
    assert oracle.round_to_f16([65519.0])[0] == 65504.0
