"""Python binding of libw4a16 (asymmetric group-128 int4 weights, fused W4A16 products on gfx950).

Argument marshalling only: every step of quantization, layout and the products
runs in the HIP kernels of ``libw4a16.so``.  PyTorch supplies device memory and
the current stream.  There is no fallback: if the library is missing or the
device is not gfx950 the calls raise.

The names mirror the C entry points declared in ``include/w4a16.h``.
"""

from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "W4Error", "lib", "declared_symbols",
    "w4_quantize", "w4_quantize_symmetric", "w4_prepared_bytes", "w4_prepare", "w4_unprepare",
    "w4_gemv", "w4_gemm_workspace_bytes", "w4_gemm", "w4_gemm_noalloc", "GEMM_NOALLOC_MAX_WORKSPACE",
    "w4_status_string", "w4_last_hip_error", "w4_format_version", "w4_stream_read",
    "w4_fp8_quantize_rows", "w4_fp8_gemm", "w4_int8_quantize_rows", "w4_int8_gemm",
    "W4Format", "w4_zeros_bytes", "w4_quantize_fmt", "w4_prepared_bytes_fmt", "w4_prepare_fmt",
    "w4_unprepare_fmt", "w4_gemv_fmt",
    "W4_OK", "W4_F32", "W4_BF16", "GROUP",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "w4a16.h")

GROUP = 128
W4_OK = 0
W4_F32 = 0
W4_BF16 = 1
GEMM_NOALLOC_MAX_WORKSPACE = 16 << 20
STATUS_NONFINITE = 1
STATUS_SCALE_OVERFLOW = 2
STATUS_SCALE_ZERO = 4

_lib = None


class W4Format(ctypes.Structure):
    """w4_format: group (32, 64, 128), scale_bf16 (0/1), zero_bits (4/8), symmetric (0/1)."""

    _fields_ = [("group", ctypes.c_int32), ("scale_bf16", ctypes.c_int32),
                ("zero_bits", ctypes.c_int32), ("symmetric", ctypes.c_int32)]

    @classmethod
    def make(cls, group=128, scale_bf16=False, zero_bits=8, symmetric=False):
        return cls(int(group), int(bool(scale_bf16)), int(zero_bits), int(bool(symmetric)))


class W4Error(RuntimeError):
    """A libw4a16 call returned a non-OK status."""

    def __init__(self, status: int, where: str):
        msg = _status_text(status)
        if status == 8:  # W4_ERR_HIP
            msg += ": " + w4_last_hip_error()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libw4a16.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m dequant_gemv_w4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    i32 = ctypes.c_int
    L.w4_quantize.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, vp]
    L.w4_quantize.restype = i32
    L.w4_quantize_symmetric.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp, vp]
    L.w4_quantize_symmetric.restype = i32
    L.w4_prepared_bytes.argtypes = [i64, i64]
    L.w4_prepared_bytes.restype = sz
    L.w4_prepare.argtypes = [vp, vp, vp, i64, i64, vp, sz, vp]
    L.w4_prepare.restype = i32
    L.w4_unprepare.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    L.w4_unprepare.restype = i32
    L.w4_gemv.argtypes = [vp, i64, i64, vp, i32, i64, vp, i32, vp]
    L.w4_gemv.restype = i32
    L.w4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    L.w4_gemm_workspace_bytes.restype = sz
    L.w4_gemm.argtypes = [vp, i64, i64, vp, i64, vp, i32, vp, sz, vp]
    L.w4_gemm.restype = i32
    L.w4_gemm_noalloc.argtypes = [vp, i64, i64, vp, i64, vp, i32, vp]
    L.w4_gemm_noalloc.restype = i32
    L.w4_status_string.argtypes = [i32]
    L.w4_status_string.restype = ctypes.c_char_p
    L.w4_last_hip_error.argtypes = []
    L.w4_last_hip_error.restype = ctypes.c_char_p
    L.w4_format_version.argtypes = []
    L.w4_format_version.restype = i32
    L.w4_stream_read.argtypes = [vp, sz, vp, vp]
    L.w4_stream_read.restype = i32
    L.w4_fp8_quantize_rows.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp]
    L.w4_fp8_quantize_rows.restype = i32
    L.w4_fp8_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, i32, vp]
    L.w4_fp8_gemm.restype = i32
    L.w4_int8_quantize_rows.argtypes = [vp, i32, i64, i64, vp, vp, vp, vp]
    L.w4_int8_quantize_rows.restype = i32
    L.w4_int8_gemm.argtypes = [vp, vp, i64, vp, vp, i64, i64, vp, i32, vp]
    L.w4_int8_gemm.restype = i32
    fp = ctypes.POINTER(W4Format)
    L.w4_zeros_bytes.argtypes = [i64, i64, fp]
    L.w4_zeros_bytes.restype = sz
    L.w4_quantize_fmt.argtypes = [vp, i32, i64, i64, fp, vp, vp, vp, vp, vp]
    L.w4_quantize_fmt.restype = i32
    L.w4_prepared_bytes_fmt.argtypes = [i64, i64, fp]
    L.w4_prepared_bytes_fmt.restype = sz
    L.w4_prepare_fmt.argtypes = [vp, vp, vp, i64, i64, fp, vp, sz, vp]
    L.w4_prepare_fmt.restype = i32
    L.w4_unprepare_fmt.argtypes = [vp, i64, i64, fp, vp, vp, vp, vp]
    L.w4_unprepare_fmt.restype = i32
    L.w4_gemv_fmt.argtypes = [vp, i64, i64, fp, vp, i32, i64, vp, i32, vp]
    L.w4_gemv_fmt.restype = i32
    del u32
    _lib = L
    return L


def declared_symbols() -> list[str]:
    """Function names declared in include/w4a16.h."""
    with open(HEADER_PATH) as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_[a-z0-9_]+)\s*\(", text)))


def _status_text(status: int) -> str:
    return lib().w4_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != W4_OK:
        raise W4Error(status, where)


def _stream(t) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _require(t, dtype, shape, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# --------------------------------------------------------------------------
# Entry points
# --------------------------------------------------------------------------

def w4_status_string(status: int) -> str:
    return _status_text(status)


def w4_last_hip_error() -> str:
    return lib().w4_last_hip_error().decode()


def w4_format_version() -> int:
    return int(lib().w4_format_version())


def w4_stream_read(buf, sink) -> None:
    """Measurement probe: read every byte of the device tensor ``buf`` once and discard it
    (``sink``: an int32 device tensor the kernel may overwrite)."""
    import torch
    _require(sink, torch.int32, None, "sink")
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _check(lib().w4_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                _stream(buf)), "w4_stream_read")


def w4_prepared_bytes(N: int, K: int) -> int:
    return int(lib().w4_prepared_bytes(int(N), int(K)))


def w4_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().w4_gemm_workspace_bytes(int(M), int(N), int(K)))


def w4_quantize(W, packed=None, scales=None, zeros=None, status=None):
    """Quantize W [N, K] (float32 or bfloat16, on the GPU).

    Returns (packed uint8 [N, K/2], scales float16 [N, K/128], zeros uint8 [N, K/128]).
    ``status`` may be an int32 tensor of one element; W4 status bits are OR-ed into it.
    """
    return _quantize("w4_quantize", W, packed, scales, zeros, status)


def w4_quantize_symmetric(W, packed=None, scales=None, zeros=None, status=None):
    """Symmetric variant (step max|w|/7, halves to even), same arrays; every zero is 8."""
    return _quantize("w4_quantize_symmetric", W, packed, scales, zeros, status)


def _quantize(fn_name, W, packed, scales, zeros, status):
    import torch
    _require(W, (torch.float32, torch.bfloat16), None, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    kg = K // GROUP
    dev = W.device
    if packed is None:
        packed = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(N, kg, dtype=torch.float16, device=dev)
    if zeros is None:
        zeros = torch.empty(N, kg, dtype=torch.uint8, device=dev)
    _require(packed, torch.uint8, (N, K // 2), "packed")
    _require(scales, torch.float16, (N, kg), "scales")
    _require(zeros, torch.uint8, (N, kg), "zeros")
    st_ptr = ctypes.c_void_p(None)
    if status is not None:
        _require(status, (torch.int32,), None, "status")
        st_ptr = _ptr(status)
    wt = W4_BF16 if W.dtype == torch.bfloat16 else W4_F32
    fn = getattr(lib(), fn_name)
    _check(fn(_ptr(W), wt, N, K, _ptr(packed), _ptr(scales), _ptr(zeros), st_ptr, _stream(W)),
           fn_name)
    return packed, scales, zeros


def w4_prepare(packed, scales, zeros, prepared=None):
    """Kernel layout of the canonical arrays; returns a uint8 tensor of w4_prepared_bytes(N, K)."""
    import torch
    _require(packed, torch.uint8, None, "packed")
    N, Kh = packed.shape
    K = 2 * Kh
    _require(scales, torch.float16, (N, K // GROUP), "scales")
    _require(zeros, torch.uint8, (N, K // GROUP), "zeros")
    nbytes = w4_prepared_bytes(N, K)
    if prepared is None:
        prepared = torch.empty(nbytes, dtype=torch.uint8, device=packed.device)
    _require(prepared, torch.uint8, None, "prepared")
    _check(lib().w4_prepare(_ptr(packed), _ptr(scales), _ptr(zeros), N, K, _ptr(prepared),
                            prepared.numel(), _stream(packed)), "w4_prepare")
    return prepared


def w4_unprepare(prepared, N: int, K: int):
    """Inverse of w4_prepare: returns (packed, scales, zeros)."""
    import torch
    _require(prepared, torch.uint8, None, "prepared")
    if prepared.numel() < w4_prepared_bytes(N, K):
        raise ValueError("prepared buffer too small")
    dev = prepared.device
    packed = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(N, K // GROUP, dtype=torch.float16, device=dev)
    zeros = torch.empty(N, K // GROUP, dtype=torch.uint8, device=dev)
    _check(lib().w4_unprepare(_ptr(prepared), N, K, _ptr(packed), _ptr(scales), _ptr(zeros),
                              _stream(prepared)), "w4_unprepare")
    return packed, scales, zeros


def w4_gemv(prepared, N: int, K: int, x, y=None, out_dtype=None):
    """y [M, N] = x [M, K] @ w_hat^T for 1 <= M <= 16 (x bfloat16 or float32)."""
    import torch
    _require(prepared, torch.uint8, None, "prepared")
    _require(x, (torch.bfloat16, torch.float32), None, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    if out_dtype is None:
        out_dtype = y.dtype if y is not None else torch.float32
    if y is None:
        y = torch.empty(M, N, dtype=out_dtype, device=x.device)
    _require(y, (torch.float32, torch.bfloat16), (M, N), "y")
    xt = W4_F32 if x.dtype == torch.float32 else W4_BF16
    yt = W4_F32 if y.dtype == torch.float32 else W4_BF16
    _check(lib().w4_gemv(_ptr(prepared), N, K, _ptr(x), xt, M, _ptr(y), yt, _stream(x)),
           "w4_gemv")
    return y


def _fmt(fmt) -> W4Format:
    if isinstance(fmt, W4Format):
        return fmt
    if isinstance(fmt, dict):
        return W4Format.make(**fmt)
    return W4Format.make(*fmt)


def w4_zeros_bytes(N: int, K: int, fmt) -> int:
    f = _fmt(fmt)
    return int(lib().w4_zeros_bytes(int(N), int(K), ctypes.byref(f)))


def w4_prepared_bytes_fmt(N: int, K: int, fmt) -> int:
    f = _fmt(fmt)
    return int(lib().w4_prepared_bytes_fmt(int(N), int(K), ctypes.byref(f)))


def w4_quantize_fmt(W, fmt, status=None):
    """Quantize W [N, K] (float32 or bfloat16) in format ``fmt`` (a W4Format, a dict of its
    fields or a tuple).  Returns (packed uint8 [N, K/2], scales [N, K/group] float16 or
    bfloat16, zeros uint8 [N, K/group] or [w4_zeros_bytes] for 4-bit zeros)."""
    import torch
    f = _fmt(fmt)
    _require(W, (torch.float32, torch.bfloat16), None, "W")
    if W.dim() != 2:
        raise ValueError("W must be 2-D")
    N, K = W.shape
    if f.group not in (32, 64, 128) or K % f.group:
        raise ValueError("K must be a multiple of the group size (32, 64 or 128)")
    kg = K // f.group
    dev = W.device
    packed = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(N, kg, dtype=torch.bfloat16 if f.scale_bf16 else torch.float16, device=dev)
    nz = w4_zeros_bytes(N, K, f)
    zeros = torch.empty((N, kg) if f.zero_bits == 8 else (max(nz, 1),), dtype=torch.uint8, device=dev)
    st_ptr = ctypes.c_void_p(None)
    if status is not None:
        _require(status, (torch.int32,), None, "status")
        st_ptr = _ptr(status)
    wt = W4_BF16 if W.dtype == torch.bfloat16 else W4_F32
    _check(lib().w4_quantize_fmt(_ptr(W), wt, N, K, ctypes.byref(f), _ptr(packed), _ptr(scales),
                                 _ptr(zeros), st_ptr, _stream(W)), "w4_quantize_fmt")
    return packed, scales, zeros


def w4_prepare_fmt(packed, scales, zeros, fmt, prepared=None):
    """Kernel layout of a format's arrays; returns a uint8 tensor of w4_prepared_bytes_fmt."""
    import torch
    f = _fmt(fmt)
    _require(packed, torch.uint8, None, "packed")
    N, Kh = packed.shape
    K = 2 * Kh
    _require(scales, torch.bfloat16 if f.scale_bf16 else torch.float16, (N, K // f.group), "scales")
    _require(zeros, torch.uint8, None, "zeros")
    if zeros.numel() < w4_zeros_bytes(N, K, f):
        raise ValueError("zeros too small for the format")
    nbytes = w4_prepared_bytes_fmt(N, K, f)
    if prepared is None:
        prepared = torch.empty(nbytes, dtype=torch.uint8, device=packed.device)
    _require(prepared, torch.uint8, None, "prepared")
    _check(lib().w4_prepare_fmt(_ptr(packed), _ptr(scales), _ptr(zeros), N, K, ctypes.byref(f),
                                _ptr(prepared), prepared.numel(), _stream(packed)),
           "w4_prepare_fmt")
    return prepared


def w4_unprepare_fmt(prepared, N: int, K: int, fmt):
    """Inverse of w4_prepare_fmt: returns (packed, scales, zeros)."""
    import torch
    f = _fmt(fmt)
    _require(prepared, torch.uint8, None, "prepared")
    if prepared.numel() < w4_prepared_bytes_fmt(N, K, f):
        raise ValueError("prepared buffer too small")
    dev = prepared.device
    kg = K // f.group
    packed = torch.empty(N, K // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(N, kg, dtype=torch.bfloat16 if f.scale_bf16 else torch.float16, device=dev)
    nz = w4_zeros_bytes(N, K, f)
    zeros = torch.empty((N, kg) if f.zero_bits == 8 else (max(nz, 1),), dtype=torch.uint8, device=dev)
    _check(lib().w4_unprepare_fmt(_ptr(prepared), N, K, ctypes.byref(f), _ptr(packed),
                                  _ptr(scales), _ptr(zeros), _stream(prepared)), "w4_unprepare_fmt")
    return packed, scales, zeros


def w4_gemv_fmt(prepared, N: int, K: int, fmt, x, y=None, out_dtype=None):
    """w4_gemv on the prepared layout of format ``fmt``."""
    import torch
    f = _fmt(fmt)
    _require(prepared, torch.uint8, None, "prepared")
    _require(x, (torch.bfloat16, torch.float32), None, "x")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    if out_dtype is None:
        out_dtype = y.dtype if y is not None else torch.float32
    if y is None:
        y = torch.empty(M, N, dtype=out_dtype, device=x.device)
    _require(y, (torch.float32, torch.bfloat16), (M, N), "y")
    xt = W4_F32 if x.dtype == torch.float32 else W4_BF16
    yt = W4_F32 if y.dtype == torch.float32 else W4_BF16
    _check(lib().w4_gemv_fmt(_ptr(prepared), N, K, ctypes.byref(f), _ptr(x), xt, M, _ptr(y), yt,
                             _stream(x)), "w4_gemv_fmt")
    return y


def w4_gemm(prepared, N: int, K: int, X, Y=None, out_dtype=None, workspace=None):
    """Y [M, N] = X [M, K] (bfloat16) @ w_hat^T on MFMA."""
    import torch
    _require(prepared, torch.uint8, None, "prepared")
    _require(X, torch.bfloat16, None, "X")
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X must be [M, K]")
    if out_dtype is None:
        out_dtype = Y.dtype if Y is not None else torch.float32
    if Y is None:
        Y = torch.empty(M, N, dtype=out_dtype, device=X.device)
    _require(Y, (torch.float32, torch.bfloat16), (M, N), "Y")
    need = w4_gemm_workspace_bytes(M, N, K)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_ptr = _ptr(workspace) if workspace is not None else ctypes.c_void_p(None)
    ws_len = workspace.numel() if workspace is not None else 0
    yt = W4_F32 if Y.dtype == torch.float32 else W4_BF16
    _check(lib().w4_gemm(_ptr(prepared), N, K, _ptr(X), M, _ptr(Y), yt, ws_ptr, ws_len,
                         _stream(X)), "w4_gemm")
    return Y


def w4_gemm_noalloc(prepared, N: int, K: int, X, Y):
    """w4_gemm into a caller's Y [M, N] with the library's own fixed device workspace.

    The C call allocates nothing; calls that may overlap on one GPU race (they share
    that GPU's workspace)."""
    import torch
    _require(prepared, torch.uint8, None, "prepared")
    _require(X, torch.bfloat16, None, "X")
    M = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("X must be [M, K]")
    _require(Y, (torch.float32, torch.bfloat16), (M, N), "Y")
    yt = W4_F32 if Y.dtype == torch.float32 else W4_BF16
    _check(lib().w4_gemm_noalloc(_ptr(prepared), N, K, _ptr(X), M, _ptr(Y), yt, _stream(X)),
           "w4_gemm_noalloc")
    return Y


# --------------------------------------------------------------------------
# W8A8 in FP8 E4M3 (prefill): per-row quantization and the product
# --------------------------------------------------------------------------

def w4_fp8_quantize_rows(A, codes=None, scales=None, status=None):
    """Per-row E4M3 codes [rows, K] uint8 and binary32 scales [rows] of a 2-D binary32 or
    bfloat16 device tensor (optional preallocated outputs, optional int32 status word)."""
    import torch
    _require(A, (torch.float32, torch.bfloat16), None, "A")
    if A.dim() != 2 or not A.is_contiguous():
        raise ValueError("A must be a contiguous [rows, K] tensor")
    rows, k = A.shape
    if codes is None:
        codes = torch.empty(rows, k, dtype=torch.uint8, device=A.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=A.device)
    _require(codes, torch.uint8, (rows, k), "codes")
    _require(scales, torch.float32, (rows,), "scales")
    st = ctypes.c_void_p(None)
    if status is not None:
        _require(status, torch.int32, None, "status")
        st = _ptr(status)
    _check(lib().w4_fp8_quantize_rows(_ptr(A), W4_F32 if A.dtype == torch.float32 else W4_BF16,
                                      rows, k, _ptr(codes), _ptr(scales), st, _stream(A)),
           "w4_fp8_quantize_rows")
    return codes, scales


def w4_fp8_gemm(xq, sx, wq, sw, Y=None, out_dtype=None):
    """Y [M, N] = sx[m] sw[n] sum_k value(xq[m, k]) value(wq[n, k])."""
    import torch
    _require(xq, torch.uint8, None, "xq")
    _require(wq, torch.uint8, None, "wq")
    m, k = xq.shape
    n, k2 = wq.shape
    if k2 != k:
        raise ValueError("xq and wq must have the same K")
    _require(sx, torch.float32, (m,), "sx")
    _require(sw, torch.float32, (n,), "sw")
    if Y is None:
        Y = torch.empty(m, n, dtype=out_dtype or torch.float32, device=xq.device)
    _require(Y, (torch.float32, torch.bfloat16), (m, n), "Y")
    _check(lib().w4_fp8_gemm(_ptr(xq), _ptr(sx), m, _ptr(wq), _ptr(sw), n, k, _ptr(Y),
                             W4_F32 if Y.dtype == torch.float32 else W4_BF16, _stream(xq)),
           "w4_fp8_gemm")
    return Y


def w4_int8_quantize_rows(A, codes=None, scales=None, status=None):
    """Per-row symmetric INT8 codes [rows, K] int8 and binary32 steps [rows] of a 2-D
    binary32 or bfloat16 device tensor."""
    import torch
    _require(A, (torch.float32, torch.bfloat16), None, "A")
    if A.dim() != 2 or not A.is_contiguous():
        raise ValueError("A must be a contiguous [rows, K] tensor")
    rows, k = A.shape
    if codes is None:
        codes = torch.empty(rows, k, dtype=torch.int8, device=A.device)
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=A.device)
    _require(codes, torch.int8, (rows, k), "codes")
    _require(scales, torch.float32, (rows,), "scales")
    st = ctypes.c_void_p(None)
    if status is not None:
        _require(status, torch.int32, None, "status")
        st = _ptr(status)
    _check(lib().w4_int8_quantize_rows(_ptr(A), W4_F32 if A.dtype == torch.float32 else W4_BF16,
                                       rows, k, _ptr(codes), _ptr(scales), st, _stream(A)),
           "w4_int8_quantize_rows")
    return codes, scales


def w4_int8_gemm(xq, sx, wq, sw, Y=None, out_dtype=None):
    """Y [M, N] = sx[m] sw[n] sum_k xq[m, k] wq[n, k] (int8 codes, exact int32 sums)."""
    import torch
    _require(xq, torch.int8, None, "xq")
    _require(wq, torch.int8, None, "wq")
    m, k = xq.shape
    n, k2 = wq.shape
    if k2 != k:
        raise ValueError("xq and wq must have the same K")
    _require(sx, torch.float32, (m,), "sx")
    _require(sw, torch.float32, (n,), "sw")
    if Y is None:
        Y = torch.empty(m, n, dtype=out_dtype or torch.float32, device=xq.device)
    _require(Y, (torch.float32, torch.bfloat16), (m, n), "Y")
    _check(lib().w4_int8_gemm(_ptr(xq), _ptr(sx), m, _ptr(wq), _ptr(sw), n, k, _ptr(Y),
                              W4_F32 if Y.dtype == torch.float32 else W4_BF16, _stream(xq)),
           "w4_int8_gemm")
    return Y
