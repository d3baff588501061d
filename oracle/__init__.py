"""CPU oracle for the FP8 (OCP e4m3fn) weight-only linear layer.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only users. The product path never
imports this package, and this package imports nothing from the product.

The arithmetic lives in ``fp8w_oracle.c`` (plain C, OpenMP over rows); this
module marshals numpy arrays into it and adds the two output roundings used for
reporting. Sources, by page title and section:

* "FP8 weight-only (precision: fp8_weights)", section "The contract": the
  per-output-channel scale amax/448, the round-to-nearest-even codes clamped to
  +-448, the formula y = scale[n] * sum_k x[m,k] q[n,k] + bias[n], fp32
  accumulation and one rounding to the activation dtype, the error report
  (rel_l2, worst_channel_rel_l2, underflow, crest) and the fallback through
  the dequantised weight.
* "B04 - Precision & Quantization", section "The numbers, derived rather than
  tabulated": the e4m3 field layout, its table row and the footnote on the
  single NaN pattern and the 448 maximum; section "The key insight: bf16 versus
  fp16": rounding fp32 to bf16 by adding 0x7FFF plus the kept LSB and dropping
  the low half.
* "Skill: Write an FP8 Kernel", "Required reasoning process" step 2 (amax,
  scale = amax / fp8_max, cast of x / scale) and step 7 (~1 % relative error
  against a wide reference; scale = 0 handled without a division).
* W8A8: "Skill: Write an FP8 Kernel", "Required reasoning process" steps 2, 4
  and 5 and "Correctness requirements" (per-token activation scales, fp32
  accumulation, acc * scale_x[m] * scale_w[n] in the epilogue).
* E4M3FNUZ: "B04 - Precision & Quantization", the format table's FNUZ row and
  the sections "Hardware support, and where the vendors diverge" (bias 8,
  maximum 240, 0x80 NaN, no negative zero) and the trap list (the same bits
  decode a factor of two apart; tag the format).
* Group scales along k: "B04 - Precision & Quantization", sections
  "Post-training quantization versus quantization-aware training" (one scale
  per run of g = 32 / 64 / 128 weights of a row) and "The one that matters:
  quantization is a quality decision" (per-channel -> per-group); the Day-98
  lab page's storage census ("one scale per 32": the block's max |w| / 448).
  Each group is quantized as the contract quantizes a row.

Pinned by ``tests/test_oracle_*.py`` against the values and closed forms the
pages fix (no function here is "parity unpinned").
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.o_e4m3_decode.restype = ctypes.c_double
        lib.o_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.o_e4m3_encode.restype = ctypes.c_uint8
        lib.o_e4m3_encode.argtypes = [ctypes.c_float]
        lib.o_e4m3_encode_search.restype = ctypes.c_uint8
        lib.o_e4m3_encode_search.argtypes = [ctypes.c_float]
        lib.o_encoders_compare.restype = I64
        lib.o_encoders_compare.argtypes = [ctypes.c_uint64, ctypes.c_uint64, P]
        lib.o_e4m3_encode_array.restype = None
        lib.o_e4m3_encode_array.argtypes = [P, I64, P]
        lib.o_quantize_rows.restype = ctypes.c_int
        lib.o_quantize_rows.argtypes = [P, I64, I64, P, P]
        lib.o_row_amax.restype = None
        lib.o_row_amax.argtypes = [P, I64, I64, P]
        lib.o_linear_f64.restype = None
        lib.o_linear_f64.argtypes = [P, I64, I64, P, P, P, I64, P]
        lib.o_linear_f64_sampled.restype = None
        lib.o_linear_f64_sampled.argtypes = [P, I64, P, P, P, P, P, I64, P]
        lib.o_dequantize_f64.restype = None
        lib.o_dequantize_f64.argtypes = [P, P, I64, I64, P]
        lib.o_weight_error.restype = None
        lib.o_weight_error.argtypes = [P, P, P, I64, I64, P, P, P]
        lib.o_quantize_groups.restype = ctypes.c_int
        lib.o_quantize_groups.argtypes = [P, I64, I64, I64, P, P]
        lib.o_linear_f64_groups.restype = None
        lib.o_linear_f64_groups.argtypes = [P, I64, I64, P, P, I64, P, I64, P]
        lib.o_linear_f64_groups_sampled.restype = None
        lib.o_linear_f64_groups_sampled.argtypes = [P, I64, P, P, I64, P, P, P, I64, P]
        lib.o_dequantize_groups_f64.restype = None
        lib.o_dequantize_groups_f64.argtypes = [P, P, I64, I64, I64, P]
        lib.o_weight_error_groups.restype = None
        lib.o_weight_error_groups.argtypes = [P, P, P, I64, I64, I64, P, P, P]
        lib.o_linear_w8a8_f64.restype = None
        lib.o_linear_w8a8_f64.argtypes = [P, P, I64, I64, P, P, P, I64, P]
        lib.o_fnuz_decode.restype = ctypes.c_double
        lib.o_fnuz_decode.argtypes = [ctypes.c_uint8]
        lib.o_fnuz_to_ocp.restype = None
        lib.o_fnuz_to_ocp.argtypes = [P, I64, P]
        lib.o_num_threads.restype = ctypes.c_int
        lib.o_num_threads.argtypes = []
        lib.o_set_num_threads.restype = None
        lib.o_set_num_threads.argtypes = [ctypes.c_int]
        _LIB = lib
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- codec
def decode(codes) -> np.ndarray:
    """value(c) for each e4m3fn code c (NaN for 0x7F / 0xFF)."""
    lib = _lib()
    table = np.array([lib.o_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def encode_one(t: float) -> int:
    return int(_lib().o_e4m3_encode(ctypes.c_float(t)))


def encode_search_one(t: float) -> int:
    return int(_lib().o_e4m3_encode_search(ctypes.c_float(t)))


def encode(t) -> np.ndarray:
    """Round-to-nearest-even e4m3fn codes of fp32 values (scale 1), saturating at +-448."""
    t = _c(t, np.float32)
    out = np.empty(t.shape, dtype=np.uint8)
    _lib().o_e4m3_encode_array(_p(t), t.size, _p(out))
    return out


def encoders_compare(first: int, count: int):
    """Disagreements of the two independent encoders over fp32 bit patterns
    [first, first+count), NaN patterns skipped: (count_bad, first_bad_pattern)."""
    fb = ctypes.c_uint64(0)
    bad = _lib().o_encoders_compare(first, count, ctypes.addressof(fb))
    return int(bad), int(fb.value)


# ----------------------------------------------------------------- quantizer
def quantize_rows(w):
    """Per-output-channel quantization of W [n, k] fp32: (q uint8 [n,k], scale fp32 [n], status)."""
    w = _c(w, np.float32)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.uint8)
    scale = np.empty((n,), dtype=np.float32)
    st = _lib().o_quantize_rows(_p(w), n, k, _p(q), _p(scale))
    return q, scale, int(st)


def row_amax(w) -> np.ndarray:
    w = _c(w, np.float32)
    n, k = w.shape
    out = np.empty((n,), dtype=np.float64)
    _lib().o_row_amax(_p(w), n, k, _p(out))
    return out


# ----------------------------------------------------------------- linear
def linear_f64(x, q, scale, bias=None) -> np.ndarray:
    """y[m,n] = scale[n] * sum_k x[m,k] value(q[n,k]) + bias[n], in fp64.

    x: [m, k] exact activation values (float64); bias: [n] or None."""
    x = _c(x, np.float64)
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    m, k = x.shape
    n = q.shape[0]
    assert q.shape == (n, k) and scale.shape == (n,)
    b = None if bias is None else _c(bias, np.float64)
    y = np.empty((m, n), dtype=np.float64)
    _lib().o_linear_f64(_p(x), m, k, _p(q), _p(scale), _p(b), n, _p(y))
    return y


def linear_f64_sampled(x, q, scale, bias, rows, cols) -> np.ndarray:
    """The same formula for the listed (row, channel) pairs only."""
    x = _c(x, np.float64)
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    b = None if bias is None else _c(bias, np.float64)
    k = x.shape[1]
    y = np.empty(rows.shape, dtype=np.float64)
    _lib().o_linear_f64_sampled(_p(x), k, _p(q), _p(scale), _p(b), _p(rows), _p(cols),
                                rows.size, _p(y))
    return y


def dequantize_f64(q, scale=None) -> np.ndarray:
    """value(q[n,k]) * scale[n] (or the unscaled value when scale is None), fp64."""
    q = _c(q, np.uint8)
    n, k = q.shape
    s = None if scale is None else _c(scale, np.float32)
    out = np.empty((n, k), dtype=np.float64)
    _lib().o_dequantize_f64(_p(q), _p(s), n, k, _p(out))
    return out


# ----------------------------------------------------------------- roundings
def round_to_f32(y) -> np.ndarray:
    return np.asarray(y, dtype=np.float64).astype(np.float32)


def round_bf16_bits(y32) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even: add 0x7FFF plus the
    lowest kept bit, keep the high half. NaN stays a quiet NaN."""
    u = np.ascontiguousarray(y32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(y32, dtype=np.float32))
    r[nan] = 0x7FC0
    return r


def bf16_bits_to_f64(bits) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def round_to_bf16(y) -> np.ndarray:
    """y -> fl32 -> bf16 (RNE), returned as exact float64 values."""
    return bf16_bits_to_f64(round_bf16_bits(round_to_f32(y)))


def round_to_f16(y) -> np.ndarray:
    """y -> fl32 -> fp16 (numpy's round-to-nearest-even cast), as float64; values
    at or past the overflow midpoint become +-inf."""
    with np.errstate(over="ignore"):
        return round_to_f32(y).astype(np.float16).astype(np.float64)


# ----------------------------------------------------------------- metrics
def weight_error(w, q, scale) -> dict:
    """rel_l2, worst_channel_rel_l2, underflow fraction and crest (max, median)."""
    w = _c(w, np.float32)
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    n, k = w.shape
    out = np.zeros(3, dtype=np.float64)
    ch = np.empty(n, dtype=np.float64)
    crest = np.empty(n, dtype=np.float64)
    _lib().o_weight_error(_p(w), _p(q), _p(scale), n, k, _p(out), _p(ch), _p(crest))
    return {"rel_l2": float(out[0]), "worst_channel_rel_l2": float(out[1]),
            "underflow": float(out[2]), "crest_max": float(crest.max()) if n else 0.0,
            "crest_median": float(np.median(crest)) if n else 0.0,
            "channel_rel_l2": ch}


def output_metrics(y, y_ref) -> dict:
    """Per activation row m: cosine(y[m], y_ref[m]) and ||y[m]-y_ref[m]|| / ||y_ref[m]||.
    Returns the minimum cosine and the maximum relative l2 over rows."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.sum(y * y_ref, axis=1)
    ny = np.linalg.norm(y, axis=1)
    nr = np.linalg.norm(y_ref, axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        cos = np.where((ny > 0) & (nr > 0), num / (ny * nr), np.where(ny == nr, 1.0, 0.0))
        rel = np.where(nr > 0, np.linalg.norm(y - y_ref, axis=1) / nr,
                       np.where(ny == 0, 0.0, np.inf))
    return {"min_cosine": float(cos.min()), "max_rel_l2": float(rel.max())}


# ----------------------------------------------------------------- group scales along k
def _check_group(k: int, g: int) -> None:
    if g <= 0 or k % g != 0:
        raise ValueError(f"group size {g} must divide k = {k}")


def quantize_groups(w, g: int):
    """One scale per run of g weights of a row: (q uint8 [n,k], scale fp32 [n, k/g], status)."""
    w = _c(w, np.float32)
    n, k = w.shape
    _check_group(k, g)
    q = np.empty((n, k), dtype=np.uint8)
    scale = np.empty((n, k // g), dtype=np.float32)
    st = _lib().o_quantize_groups(_p(w), n, k, g, _p(q), _p(scale))
    return q, scale, int(st)


def linear_f64_groups(x, q, scale, g: int, bias=None) -> np.ndarray:
    """y[m,n] = sum_j scale[n,j] * sum_{i<g} x[m,jg+i] value(q[n,jg+i]) + bias[n], in fp64."""
    x = _c(x, np.float64)
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    m, k = x.shape
    n = q.shape[0]
    _check_group(k, g)
    assert q.shape == (n, k) and scale.shape == (n, k // g)
    b = None if bias is None else _c(bias, np.float64)
    y = np.empty((m, n), dtype=np.float64)
    _lib().o_linear_f64_groups(_p(x), m, k, _p(q), _p(scale), g, _p(b), n, _p(y))
    return y


def linear_f64_groups_sampled(x, q, scale, g: int, bias, rows, cols) -> np.ndarray:
    """The same formula for the listed (row, channel) pairs only."""
    x = _c(x, np.float64)
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    b = None if bias is None else _c(bias, np.float64)
    k = x.shape[1]
    _check_group(k, g)
    y = np.empty(rows.shape, dtype=np.float64)
    _lib().o_linear_f64_groups_sampled(_p(x), k, _p(q), _p(scale), g, _p(b), _p(rows), _p(cols), rows.size, _p(y))
    return y


def dequantize_groups_f64(q, scale, g: int) -> np.ndarray:
    """value(q[n,k]) * scale[n, k/g], fp64."""
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    n, k = q.shape
    _check_group(k, g)
    out = np.empty((n, k), dtype=np.float64)
    _lib().o_dequantize_groups_f64(_p(q), _p(scale), g, n, k, _p(out))
    return out


def weight_error_groups(w, q, scale, g: int) -> dict:
    """rel_l2, worst_channel_rel_l2, underflow and crest with group scales."""
    w = _c(w, np.float32)
    q = _c(q, np.uint8)
    scale = _c(scale, np.float32)
    n, k = w.shape
    _check_group(k, g)
    out = np.zeros(3, dtype=np.float64)
    ch = np.empty(n, dtype=np.float64)
    crest = np.empty(n, dtype=np.float64)
    _lib().o_weight_error_groups(_p(w), _p(q), _p(scale), g, n, k, _p(out), _p(ch), _p(crest))
    return {"rel_l2": float(out[0]), "worst_channel_rel_l2": float(out[1]),
            "underflow": float(out[2]), "crest_max": float(crest.max()) if n else 0.0,
            "crest_median": float(np.median(crest)) if n else 0.0,
            "channel_rel_l2": ch}


# ----------------------------------------------------------------- W8A8
def quantize_activations(x):
    """Per-token e4m3 quantization of activations x [m, k] (their exact values):
    the row quantizer applied to the rows of x. Returns (qx, scale_x, status)."""
    return quantize_rows(np.asarray(x, dtype=np.float64).astype(np.float32))


def linear_w8a8_f64(qx, sx, qw, sw, bias=None) -> np.ndarray:
    """y[m,n] = (sum_k value(qx[m,k]) value(qw[n,k])) * sx[m] * sw[n] + bias[n], fp64."""
    qx = _c(qx, np.uint8)
    qw = _c(qw, np.uint8)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    m, k = qx.shape
    n = qw.shape[0]
    assert qw.shape == (n, k) and sx.shape == (m,) and sw.shape == (n,)
    b = None if bias is None else _c(bias, np.float64)
    y = np.empty((m, n), dtype=np.float64)
    _lib().o_linear_w8a8_f64(_p(qx), _p(sx), m, k, _p(qw), _p(sw), _p(b), n, _p(y))
    return y


# ----------------------------------------------------------------- E4M3FNUZ interop
def fnuz_decode(codes) -> np.ndarray:
    """E4M3FNUZ values (bias 8, 0x80 NaN, no negative zero) of uint8 codes, fp64."""
    c = np.asarray(codes, dtype=np.uint8)
    lib = _lib()
    return np.vectorize(lambda v: lib.o_fnuz_decode(int(v)), otypes=[np.float64])(c)


def fnuz_to_ocp(codes) -> np.ndarray:
    """OCP e4m3fn codes of the same values as the given E4M3FNUZ codes (RNE; NaN -> 0x7F)."""
    c = _c(codes, np.uint8)
    out = np.empty(c.shape, dtype=np.uint8)
    _lib().o_fnuz_to_ocp(_p(c), c.size, _p(out))
    return out


def num_threads() -> int:
    return int(_lib().o_num_threads())


def set_num_threads(n: int) -> None:
    _lib().o_set_num_threads(int(n))
