"""fp8_weight_only_amd — FP8 (OCP e4m3fn) weight-only linear layer for MI355X.

A thin ctypes binding over ``libfp8w.so`` (declared in ``include/fp8w.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks tensors, hands their device pointers and torch's current HIP stream
to the C ABI, and allocates outputs with torch (torch is plumbing here: device
memory and streams).

The raw entry points keep the C names (``fp8w_quantize``, ``fp8w_linear``,
``fp8w_linear_with_path``, ``fp8w_dequantize_fallback``, ``fp8w_linear_path``,
``fp8w_linear_workspace_bytes``, ``fp8w_status_string``) and take integers
(pointers, sizes, the stream handle). The tensor-level helpers ``quantize``,
``linear``, ``dequantize`` and the ``QuantizedLinear`` holder sit on top.

The method ("FP8 weight-only (precision: fp8_weights)", section "The
contract"): quantise once at build time with one scale per output channel,
scale = amax(|row|) / 448 and codes rounded to nearest even in e4m3 (clamped
to +-448), keep no higher-precision copy, and per call compute
y = scale[n] * sum_k x[m,k] q[n,k] + bias[n] with fp32 accumulation and one
rounding to the activation dtype.

If ``libfp8w.so`` has not been built, importing the package still works but
every call raises: there is no CPU or PyTorch fallback.
"""
import ctypes
import os

import torch

__all__ = [
    "Fp8wError", "lib_path", "load", "fp8w_quantize", "fp8w_linear", "fp8w_linear_with_path", "fp8w_linear_noalloc", "linear_noalloc", "SCRATCH_BYTES",
    "fp8w_dequantize_fallback", "fp8w_linear_path", "fp8w_linear_workspace_bytes", "fp8w_linear_with_path_workspace_bytes",
    "fp8w_linear_kernel",
    "fp8w_stream_read_probe", "fp8w_quantize_grouped", "fp8w_linear_grouped", "fp8w_linear_grouped_with_path",
    "fp8w_linear_grouped_path", "fp8w_linear_grouped_kernel", "fp8w_dequantize_grouped",
    "fp8w_linear_grouped_with_workspace", "fp8w_linear_grouped_workspace_bytes", "grouped_workspace_bytes",
    "quantize_grouped", "linear_grouped", "dequantize_grouped", "fp8w_fnuz_to_ocp", "fnuz_to_ocp", "ocp_codes",
    "fp8w_quantize_activations", "fp8w_gemm_w8a8", "fp8w_linear_w8a8", "fp8w_linear_w8a8_workspace_bytes",
    "fp8w_linear_w8a8_kernel", "quantize_activations", "gemm_w8a8", "linear_w8a8",
    "fp8w_status_string", "fp8w_abi_version", "quantize", "linear", "dequantize",
    "linear_path", "workspace_bytes", "QuantizedLinear",
    "BF16", "FP16", "FP32", "PATH_AUTO", "PATH_GEMV", "PATH_SKINNY", "PATH_FALLBACK", "PATH_BATCH", "EXPORTS",
]

BF16, FP16, FP32 = 0, 1, 2
SCRATCH_BYTES = 32 << 20  # FP8W_SCRATCH_BYTES: the static scratch of fp8w_linear_noalloc, per GPU
PATH_AUTO, PATH_GEMV, PATH_SKINNY, PATH_FALLBACK, PATH_BATCH = -1, 0, 1, 2, 3
SUCCESS, ERR_INVALID_VALUE, ERR_MISALIGNED, ERR_NONFINITE, ERR_WORKSPACE, ERR_HIP = range(6)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_I = ctypes.c_int

# name -> (restype, argtypes), mirroring include/fp8w.h
EXPORTS = {
    "fp8w_quantize": (_I, [_P, _I, _I64, _I64, _P, _P, _P]),
    "fp8w_linear": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "fp8w_linear_with_path": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I64, _P, _P, _SZ, _I, _P]),
    "fp8w_linear_noalloc": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I64, _P, _P]),
    "fp8w_dequantize_fallback": (_I, [_P, _P, _I64, _I64, _P, _I, _P]),
    "fp8w_linear_path": (_I, [_I64, _I64, _I64, _I, _P, _P, _P]),
    "fp8w_linear_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I, _P, _P, _P]),
    "fp8w_linear_with_path_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I, _P, _P]),
    "fp8w_linear_kernel": (ctypes.c_char_p, [_I, _I64, _I64, _I64, _I, _P, _P]),
    "fp8w_stream_read_probe": (_I, [_P, _SZ, _P, _P]),
    "fp8w_quantize_grouped": (_I, [_P, _I, _I64, _I64, _I64, _P, _P, _P]),
    "fp8w_linear_grouped": (_I, [_P, _I, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _P]),
    "fp8w_linear_grouped_with_path": (_I, [_P, _I, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _I, _P]),
    "fp8w_linear_grouped_with_workspace": (_I, [_P, _I, _I64, _I64, _P, _P, _I64, _P, _I64, _P, _P, _SZ, _I, _P]),
    "fp8w_linear_grouped_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I, _P, _P]),
    "fp8w_linear_grouped_path": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P]),
    "fp8w_linear_grouped_kernel": (ctypes.c_char_p, [_I, _I64, _I64, _I64, _I64, _I, _P, _P]),
    "fp8w_dequantize_grouped": (_I, [_P, _P, _I64, _I64, _I64, _P, _I, _P]),
    "fp8w_fnuz_to_ocp": (_I, [_P, _I64, _P, _P]),
    "fp8w_quantize_activations": (_I, [_P, _I, _I64, _I64, _P, _P, _P]),
    "fp8w_gemm_w8a8": (_I, [_P, _P, _I64, _I64, _P, _P, _P, _I64, _P, _I, _P]),
    "fp8w_linear_w8a8_workspace_bytes": (_SZ, [_I64, _I64]),
    "fp8w_linear_w8a8": (_I, [_P, _I, _I64, _I64, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "fp8w_linear_w8a8_kernel": (ctypes.c_char_p, [_I64, _I64, _I64]),
    "fp8w_status_string": (ctypes.c_char_p, [_I]),
    "fp8w_last_hip_error": (_I, []),
    "fp8w_abi_version": (_I, []),
}


class Fp8wError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = fp8w_status_string(status)
        if status == ERR_HIP:
            msg += f" (hipError {load().fp8w_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


def lib_path() -> str:
    return os.path.join(_HERE, "libfp8w.so")


def load():
    """Load libfp8w.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()'); "
                               "there is no non-HIP implementation")
        lib = ctypes.CDLL(p)
        for name, (res, args) in EXPORTS.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _LIB = lib
    return _LIB


# ------------------------------------------------------------------ raw C entry points
def fp8w_quantize(w, w_dtype, n, k, q, scale, stream) -> int:
    return load().fp8w_quantize(w, w_dtype, n, k, q, scale, stream)


def fp8w_linear(x, act_dtype, m, k, q, scale, bias, n, y, workspace, workspace_bytes, stream) -> int:
    return load().fp8w_linear(x, act_dtype, m, k, q, scale, bias, n, y, workspace, workspace_bytes, stream)


def fp8w_linear_with_path(x, act_dtype, m, k, q, scale, bias, n, y, workspace, workspace_bytes, path,
                          stream) -> int:
    return load().fp8w_linear_with_path(x, act_dtype, m, k, q, scale, bias, n, y, workspace, workspace_bytes,
                                        path, stream)


def fp8w_dequantize_fallback(q, scale, n, k, out, out_dtype, stream) -> int:
    return load().fp8w_dequantize_fallback(q, scale, n, k, out, out_dtype, stream)


def fp8w_linear_path(m, n, k, act_dtype, x, q, y) -> int:
    return load().fp8w_linear_path(m, n, k, act_dtype, x, q, y)


def fp8w_linear_workspace_bytes(m, n, k, act_dtype, x, q, y) -> int:
    return load().fp8w_linear_workspace_bytes(m, n, k, act_dtype, x, q, y)


def fp8w_linear_noalloc(x, act_dtype, m, k, q, scale, bias, n, y, stream) -> int:
    return load().fp8w_linear_noalloc(x, act_dtype, m, k, q, scale, bias, n, y, stream)


def fp8w_linear_with_path_workspace_bytes(path, m, n, k, act_dtype, x, q) -> int:
    return load().fp8w_linear_with_path_workspace_bytes(path, m, n, k, act_dtype, x, q)


def fp8w_linear_kernel(path, m, n, k, act_dtype, x, q):
    """Name of the kernel `path` launches for these sizes (None if invalid)."""
    r = load().fp8w_linear_kernel(path, m, n, k, act_dtype, x, q)
    return r.decode() if r is not None else None


def fp8w_stream_read_probe(p, nbytes, sink, stream) -> int:
    return load().fp8w_stream_read_probe(p, nbytes, sink, stream)


def fp8w_quantize_grouped(w, w_dtype, n, k, group, q, scale, stream) -> int:
    return load().fp8w_quantize_grouped(w, w_dtype, n, k, group, q, scale, stream)


def fp8w_linear_grouped(x, act_dtype, m, k, q, scale, group, bias, n, y, stream) -> int:
    return load().fp8w_linear_grouped(x, act_dtype, m, k, q, scale, group, bias, n, y, stream)


def fp8w_linear_grouped_with_path(x, act_dtype, m, k, q, scale, group, bias, n, y, path, stream) -> int:
    return load().fp8w_linear_grouped_with_path(x, act_dtype, m, k, q, scale, group, bias, n, y, path, stream)


def fp8w_linear_grouped_with_workspace(x, act_dtype, m, k, q, scale, group, bias, n, y, workspace, workspace_bytes,
                                       path, stream) -> int:
    return load().fp8w_linear_grouped_with_workspace(x, act_dtype, m, k, q, scale, group, bias, n, y, workspace,
                                                     workspace_bytes, path, stream)


def fp8w_linear_grouped_workspace_bytes(m, n, k, group, act_dtype, x, q) -> int:
    return load().fp8w_linear_grouped_workspace_bytes(m, n, k, group, act_dtype, x, q)


def fp8w_linear_grouped_path(m, n, k, group, act_dtype, x, q) -> int:
    return load().fp8w_linear_grouped_path(m, n, k, group, act_dtype, x, q)


def fp8w_linear_grouped_kernel(path, m, n, k, group, act_dtype, x, q):
    r = load().fp8w_linear_grouped_kernel(path, m, n, k, group, act_dtype, x, q)
    return r.decode() if r is not None else None


def fp8w_dequantize_grouped(q, scale, group, n, k, out, out_dtype, stream) -> int:
    return load().fp8w_dequantize_grouped(q, scale, group, n, k, out, out_dtype, stream)


def fp8w_fnuz_to_ocp(src, count, dst, stream) -> int:
    return load().fp8w_fnuz_to_ocp(src, count, dst, stream)


def fp8w_quantize_activations(x, act_dtype, m, k, qx, sx, stream) -> int:
    return load().fp8w_quantize_activations(x, act_dtype, m, k, qx, sx, stream)


def fp8w_gemm_w8a8(qx, sx, m, k, qw, sw, bias, n, y, out_dtype, stream) -> int:
    return load().fp8w_gemm_w8a8(qx, sx, m, k, qw, sw, bias, n, y, out_dtype, stream)


def fp8w_linear_w8a8_workspace_bytes(m, k) -> int:
    return load().fp8w_linear_w8a8_workspace_bytes(m, k)


def fp8w_linear_w8a8(x, act_dtype, m, k, qw, sw, bias, n, y, workspace, workspace_bytes, stream) -> int:
    return load().fp8w_linear_w8a8(x, act_dtype, m, k, qw, sw, bias, n, y, workspace, workspace_bytes, stream)


def fp8w_linear_w8a8_kernel(m, n, k):
    r = load().fp8w_linear_w8a8_kernel(m, n, k)
    return r.decode() if r is not None else None


def fp8w_status_string(status) -> str:
    return load().fp8w_status_string(status).decode()


def fp8w_abi_version() -> int:
    return load().fp8w_abi_version()


# ------------------------------------------------------------------ tensor helpers
_DT = {torch.bfloat16: BF16, torch.float16: FP16, torch.float32: FP32}


def _dtype_code(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}")
    return _DT[t]


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(st: int, where: str) -> None:
    if st != SUCCESS:
        raise Fp8wError(st, where)


def quantize(w: torch.Tensor):
    """Per-output-channel e4m3 quantization of a [n, k] weight (fp32, bf16 or fp16).

    Returns (q uint8 [n, k], scale fp32 [n]). Raises Fp8wError (status
    ERR_NONFINITE) on NaN / inf weights."""
    if w.dim() != 2:
        raise ValueError("w must be [n, k]")
    n, k = w.shape
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n,), dtype=torch.float32, device=w.device)
    st = fp8w_quantize(_dev(w, "w") if w.numel() else 0, _dtype_code(w.dtype), n, k,
                       q.data_ptr() if q.numel() else 0, scale.data_ptr() if n else 0, _stream(w.device))
    _check(st, "fp8w_quantize")
    return q, scale


def linear_path(x: torch.Tensor, q: torch.Tensor, y: torch.Tensor = None) -> int:
    m, k = x.shape
    return fp8w_linear_path(m, q.shape[0], k, _dtype_code(x.dtype), x.data_ptr(), q.data_ptr(),
                            0 if y is None else y.data_ptr())


def workspace_bytes(x: torch.Tensor, q: torch.Tensor, y: torch.Tensor = None) -> int:
    m, k = x.shape
    return fp8w_linear_workspace_bytes(m, q.shape[0], k, _dtype_code(x.dtype), x.data_ptr(), q.data_ptr(),
                                       0 if y is None else y.data_ptr())


def linear(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, bias: torch.Tensor = None,
           out: torch.Tensor = None, workspace: torch.Tensor = None, path: int = PATH_AUTO) -> torch.Tensor:
    """y = scale[n] * sum_k x[m,k] value(q[n,k]) + bias[n], rounded once to x.dtype.

    x: [m, k] bf16 / fp16; q: [n, k] uint8 codes; scale: [n] fp32; bias: [n]
    of x.dtype or None. ``workspace`` (any device tensor) is what the C ABI
    calls workspace: needed on the fallback path, used for a k split on some
    skinny and batch shapes. When it is None and the call uses one, one of
    fp8w_linear_workspace_bytes is allocated here with torch; an empty tensor
    makes such shapes take their single-pass plan."""
    if x.dim() != 2 or q.dim() != 2 or q.dtype != torch.uint8 or scale.dtype != torch.float32:
        raise ValueError("expected x [m,k], q uint8 [n,k], scale fp32 [n]")
    m, k = x.shape
    n = q.shape[0]
    if q.shape[1] != k or scale.shape != (n,):
        raise ValueError("shape mismatch between x, q and scale")
    if bias is not None and (bias.shape != (n,) or bias.dtype != x.dtype):
        raise ValueError("bias must be [n] in the activation dtype")
    act = _dtype_code(x.dtype)
    if act == FP32:
        raise TypeError("activations must be bf16 or fp16")
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    elif out.shape != (m, n) or out.dtype != x.dtype:
        raise ValueError("out must be [m, n] in the activation dtype")
    xp = _dev(x, "x") if x.numel() else 0
    qp = _dev(q, "q") if q.numel() else 0
    sp = _dev(scale, "scale") if n else 0
    bp = _dev(bias, "bias") if bias is not None and n else 0
    yp = _dev(out, "out") if out.numel() else 0
    need = fp8w_linear_with_path_workspace_bytes(path, m, n, k, act, xp, qp)
    if need and workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    wp = _dev(workspace, "workspace") if workspace is not None and workspace.numel() else 0
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = fp8w_linear_with_path(xp, act, m, k, qp, sp, bp, n, yp, wp, wb, path, _stream(x.device))
    _check(st, "fp8w_linear")
    return out


def linear_noalloc(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, bias: torch.Tensor = None,
                   out: torch.Tensor = None) -> torch.Tensor:
    """``linear`` through fp8w_linear_noalloc: any workspace the call uses is the
    library's static per-GPU scratch, so with ``out`` given nothing is allocated.
    Calls that may overlap on one GPU must not be made (they share the scratch)."""
    if x.dim() != 2 or q.dim() != 2 or q.dtype != torch.uint8 or scale.dtype != torch.float32:
        raise ValueError("expected x [m,k], q uint8 [n,k], scale fp32 [n]")
    m, k = x.shape
    n = q.shape[0]
    if q.shape[1] != k or scale.shape != (n,):
        raise ValueError("shape mismatch between x, q and scale")
    if bias is not None and (bias.shape != (n,) or bias.dtype != x.dtype):
        raise ValueError("bias must be [n] in the activation dtype")
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    elif out.shape != (m, n) or out.dtype != x.dtype:
        raise ValueError("out must be [m, n] in the activation dtype")
    st = fp8w_linear_noalloc(_dev(x, "x") if x.numel() else 0, _dtype_code(x.dtype), m, k,
                             _dev(q, "q") if q.numel() else 0, _dev(scale, "scale") if n else 0,
                             _dev(bias, "bias") if bias is not None and n else 0, n,
                             _dev(out, "out") if out.numel() else 0, _stream(x.device))
    _check(st, "fp8w_linear_noalloc")
    return out


def dequantize(q: torch.Tensor, scale: torch.Tensor = None, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """value(q) * scale[:, None] in ``dtype`` (fp32: exactly q.float() * scale[:, None]),
    or the exact unscaled values when scale is None."""
    n, k = q.shape
    out = torch.empty((n, k), dtype=dtype, device=q.device)
    st = fp8w_dequantize_fallback(_dev(q, "q") if q.numel() else 0,
                                  _dev(scale, "scale") if scale is not None and n else 0,
                                  n, k, out.data_ptr() if out.numel() else 0, _dtype_code(dtype),
                                  _stream(q.device))
    _check(st, "fp8w_dequantize_fallback")
    return out


def quantize_grouped(w: torch.Tensor, group: int):
    """e4m3 quantization with one scale per run of ``group`` (32, 64 or 128)
    weights of each row of a [n, k] weight. Returns (q uint8 [n, k], scale fp32
    [n, k // group])."""
    if w.dim() != 2:
        raise ValueError("w must be [n, k]")
    n, k = w.shape
    if group <= 0 or k % group:
        raise ValueError("group must divide k")
    q = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n, k // group), dtype=torch.float32, device=w.device)
    st = fp8w_quantize_grouped(_dev(w, "w") if w.numel() else 0, _dtype_code(w.dtype), n, k, group,
                               q.data_ptr() if q.numel() else 0, scale.data_ptr() if scale.numel() else 0,
                               _stream(w.device))
    _check(st, "fp8w_quantize_grouped")
    return q, scale


def grouped_workspace_bytes(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor) -> int:
    m, k = x.shape
    group = k // scale.shape[1]
    return fp8w_linear_grouped_workspace_bytes(m, q.shape[0], k, group, _dtype_code(x.dtype), x.data_ptr(),
                                               q.data_ptr())


def linear_grouped(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, bias: torch.Tensor = None,
                   out: torch.Tensor = None, path: int = PATH_AUTO, workspace: torch.Tensor = None) -> torch.Tensor:
    """y = sum_j scale[n, j] * sum_{k in group j} x[m,k] value(q[n,k]) + bias[n],
    rounded once to x.dtype; scale is [n, k // group] (the group size follows).
    ``workspace``: used for a k split on some batch shapes (m > 32); when None
    and the call's plan splits, one of fp8w_linear_grouped_workspace_bytes is
    allocated here with torch; an empty tensor keeps the single-pass plan."""
    if x.dim() != 2 or q.dim() != 2 or q.dtype != torch.uint8 or scale.dtype != torch.float32 or scale.dim() != 2:
        raise ValueError("expected x [m,k], q uint8 [n,k], scale fp32 [n, k // group]")
    m, k = x.shape
    n = q.shape[0]
    if q.shape[1] != k or scale.shape[0] != n or scale.shape[1] == 0 or k % scale.shape[1]:
        raise ValueError("shape mismatch between x, q and scale")
    group = k // scale.shape[1]
    if bias is not None and (bias.shape != (n,) or bias.dtype != x.dtype):
        raise ValueError("bias must be [n] in the activation dtype")
    act = _dtype_code(x.dtype)
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    elif out.shape != (m, n) or out.dtype != x.dtype:
        raise ValueError("out must be [m, n] in the activation dtype")
    xp = _dev(x, "x") if x.numel() else 0
    qp = _dev(q, "q") if q.numel() else 0
    need = 0
    if path in (PATH_AUTO, PATH_BATCH) and fp8w_linear_grouped_path(m, n, k, group, act, xp, qp) == PATH_BATCH:
        need = fp8w_linear_grouped_workspace_bytes(m, n, k, group, act, xp, qp)
    if need and workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    wp = _dev(workspace, "workspace") if workspace is not None and workspace.numel() else 0
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = fp8w_linear_grouped_with_workspace(xp, act, m, k, qp, _dev(scale, "scale"), group,
                                            _dev(bias, "bias") if bias is not None and n else 0, n,
                                            _dev(out, "out") if out.numel() else 0, wp, wb, path,
                                            _stream(x.device))
    _check(st, "fp8w_linear_grouped")
    return out


def dequantize_grouped(q: torch.Tensor, scale: torch.Tensor, dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """value(q[n,k]) * scale[n, k // group] in ``dtype`` (fp32: exactly the fp32 product)."""
    n, k = q.shape
    group = k // scale.shape[1]
    out = torch.empty((n, k), dtype=dtype, device=q.device)
    st = fp8w_dequantize_grouped(_dev(q, "q"), _dev(scale, "scale"), group, n, k, out.data_ptr(),
                                 _dtype_code(dtype), _stream(q.device))
    _check(st, "fp8w_dequantize_grouped")
    return out


def quantize_activations(x: torch.Tensor):
    """Per-token e4m3 quantization of activations x [m, k] (bf16 / fp16):
    (qx uint8 [m, k], sx fp32 [m]). Asynchronous; non-finite rows get NaN scales."""
    m, k = x.shape
    qx = torch.empty((m, k), dtype=torch.uint8, device=x.device)
    sx = torch.empty((m,), dtype=torch.float32, device=x.device)
    st = fp8w_quantize_activations(_dev(x, "x") if x.numel() else 0, _dtype_code(x.dtype), m, k,
                                   qx.data_ptr() if qx.numel() else 0, sx.data_ptr() if m else 0, _stream(x.device))
    _check(st, "fp8w_quantize_activations")
    return qx, sx


def gemm_w8a8(qx: torch.Tensor, sx: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, bias: torch.Tensor = None,
              out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor = None) -> torch.Tensor:
    """y = (sum_k value(qx) value(q)) * sx[:, None] * scale[None, :] + bias, rounded once to out_dtype."""
    m, k = qx.shape
    n = q.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=qx.device)
    st = fp8w_gemm_w8a8(_dev(qx, "qx"), _dev(sx, "sx"), m, k, _dev(q, "q"), _dev(scale, "scale"),
                        _dev(bias, "bias") if bias is not None else 0, n, _dev(out, "out"),
                        _dtype_code(out.dtype), _stream(qx.device))
    _check(st, "fp8w_gemm_w8a8")
    return out


def linear_w8a8(x: torch.Tensor, q: torch.Tensor, scale: torch.Tensor, bias: torch.Tensor = None,
                out: torch.Tensor = None, workspace: torch.Tensor = None) -> torch.Tensor:
    """The W8A8 layer on bf16 / fp16 activations: per-token quantization of x
    into the workspace, then the fp8 x fp8 GEMM (see gemm_w8a8)."""
    m, k = x.shape
    n = q.shape[0]
    need = fp8w_linear_w8a8_workspace_bytes(m, k)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=x.device)
    st = fp8w_linear_w8a8(_dev(x, "x"), _dtype_code(x.dtype), m, k, _dev(q, "q"), _dev(scale, "scale"),
                          _dev(bias, "bias") if bias is not None else 0, n, _dev(out, "out"),
                          _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                          _stream(x.device))
    _check(st, "fp8w_linear_w8a8")
    return out


def fnuz_to_ocp(codes: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """OCP e4m3fn codes (uint8) of the same values as E4M3FNUZ codes (uint8 or
    torch.float8_e4m3fnuz); ``out`` may be ``codes`` itself (in place)."""
    src = codes.view(torch.uint8) if codes.dtype != torch.uint8 else codes
    if out is None:
        out = torch.empty_like(src)
    n = src.numel()
    st = fp8w_fnuz_to_ocp(_dev(src, "codes") if n else 0, n, _dev(out, "out") if n else 0, _stream(src.device))
    _check(st, "fp8w_fnuz_to_ocp")
    return out


def ocp_codes(codes: torch.Tensor) -> torch.Tensor:
    """The weight codes this library takes (OCP e4m3fn bytes), from a tensor
    whose dtype is its format tag: torch.float8_e4m3fn is viewed as bytes,
    torch.float8_e4m3fnuz is translated value for value (fnuz_to_ocp), and
    plain uint8 is taken as OCP already."""
    if codes.dtype == torch.float8_e4m3fn:
        return codes.view(torch.uint8)
    if codes.dtype == torch.float8_e4m3fnuz:
        return fnuz_to_ocp(codes)
    if codes.dtype == torch.uint8:
        return codes
    raise TypeError(f"not an e4m3 code tensor: {codes.dtype}")


class QuantizedLinear:
    """An nn.Linear-shaped layer whose weight is held only as e4m3 codes + scales.

    ``QuantizedLinear.build(weight, bias)`` quantises once; ``__call__(x)``
    runs the fp8w linear. The original weight is not kept."""

    def __init__(self, q: torch.Tensor, scale: torch.Tensor, bias: torch.Tensor = None):
        self.q, self.scale, self.bias = q, scale, bias
        self.split_sizes = [int(q.shape[0])]
        self._ws = None

    @classmethod
    def build(cls, weight: torch.Tensor, bias: torch.Tensor = None) -> "QuantizedLinear":
        q, scale = quantize(weight)
        return cls(q, scale, bias)

    @classmethod
    def build_merged(cls, weights, biases=None) -> "QuantizedLinear":
        """One layer for several that read the same input (q/k/v, gate/up): the
        weights are stacked along the output dimension and quantised once. The
        scales are per output row, so each row's codes and scale are exactly
        those of its own layer; the output's columns are the layers' outputs
        side by side (``split_sizes`` gives their widths). Biases: all or none."""
        weights = list(weights)
        if biases is not None and any(b is None for b in biases):
            raise ValueError("build_merged: give a bias for every layer or for none")
        w = torch.cat([wi.reshape(wi.shape[0], -1) for wi in weights], dim=0)
        b = None if biases is None else torch.cat(list(biases))
        layer = cls.build(w, b)
        layer.split_sizes = [int(wi.shape[0]) for wi in weights]
        return layer

    @property
    def out_features(self) -> int:
        return self.q.shape[0]

    @property
    def in_features(self) -> int:
        return self.q.shape[1]

    def __call__(self, x: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
        lead = x.shape[:-1]
        x2 = x.reshape(-1, x.shape[-1]).contiguous()
        need = workspace_bytes(x2, self.q)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.empty((need,), dtype=torch.uint8, device=x.device)
        y = linear(x2, self.q, self.scale, self.bias, out=out, workspace=self._ws if need else None)
        return y.reshape(*lead, self.out_features)
