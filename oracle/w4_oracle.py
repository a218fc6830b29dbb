"""CPU oracle for asymmetric group-wise 4-bit weight quantization and the W4A16 product.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module.  The product path
(the HIP library and its Python binding) never calls it and shares no code,
table or constant generator with it.

What it computes (page "Weight quantization", sections "How it works" and
"Code"; the affine map is also stated on "LLM Quantization Architecture in
Depth" › "Number formats, scales and granularity"):

* groups are 128 consecutive weights along the input dimension of one row;
* the group's minimum and maximum are widened so that 0 lies in the range;
* scale  = (max - min) / 15, or 1 when the widened range is empty;
* zero   = round(-min / scale), clamped to [0, 15];
* code   = clamp(round(w / scale) + zero, 0, 15);
* two codes share a byte, the even input index in the low nibble;
* the stored scale is the f32 scale rounded to fp16 (round to nearest even;
  the page sizes its format with fp16 scales), the stored zero is a byte;
* dequantized weight  w_hat = (code - zero) * scale16;
* y[m, n] = sum_k w_hat[n, k] * x[m, k], evaluated in fp64 (dequantize, then dot).

Readings where the pages are silent (each is also pinned by a test):

* ``round`` rounds halves away from zero (the page's code uses a Rust f32
  ``round``), never half-to-even;
* every step of the quantizer is one IEEE binary32 operation: a true division
  (not a reciprocal multiply), no fused multiply-add, subnormals kept;
* codes and zero come from the f32 scale; only the stored scale is fp16;
* the codes add the clamped f32 zero (not the stored byte) to the rounded
  quotient, and a NaN that reaches a byte conversion gives 0 (the page's
  ``as u8`` cast); NaN only appears when a group's range is so small that its
  f32 scale underflows to 0.  Non-finite weights are rejected.

Two independent emulations of the f32 steps are provided: ``quantize_scalar``
(pure Python: every operation in fp64 and then rounded once to binary32, which
is exact for + - * / because 53 >= 2*24 + 2) and ``quantize_ref`` (NumPy
float32 ufuncs, vectorised).  Tests check each against definitions outside this
file (exact rational arithmetic, IEEE binary16 values, brute-force searches).
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np

GROUP = 128
QMAX = 15  # 2^4 - 1


# ---------------------------------------------------------------------------
# Scalar path: pure Python, one f32 rounding per operation
# ---------------------------------------------------------------------------

def f32(v: float) -> float:
    """Round a Python float to the nearest binary32 value (ties to even), overflow to inf."""
    if v != v or v in (math.inf, -math.inf):
        return v
    try:
        return struct.unpack("<f", struct.pack("<f", v))[0]
    except OverflowError:
        return math.copysign(math.inf, v)


def ieee_div(a: float, b: float) -> float:
    """a / b with IEEE semantics for a zero divisor (Python raises instead)."""
    if b == 0.0:
        if a == 0.0 or a != a:
            return math.nan
        sign = math.copysign(1.0, a) * math.copysign(1.0, b)
        return math.copysign(math.inf, sign)
    return a / b


def round_away(t: float) -> float:
    """Nearest integer, halves away from zero.  Exact in fp64 for any binary32 input."""
    if t != t or t in (math.inf, -math.inf):
        return t
    return math.copysign(math.floor(abs(t) + 0.5), t)


def clamp_code(t: float) -> float:
    """clamp(t, 0, 15) in f32; a NaN stays NaN (as the page's f32 clamp does)."""
    if t != t:
        return t
    return min(max(t, 0.0), float(QMAX))


def to_code(t: float) -> int:
    """clamp(t, 0, 15) converted to a byte; NaN converts to 0."""
    t = clamp_code(t)
    if t != t:
        return 0
    return int(t)


def fp16_bits(v: float) -> int:
    """binary16 bit pattern of v (round to nearest even; overflow to +-inf)."""
    try:
        return struct.unpack("<H", struct.pack("<e", v))[0]
    except OverflowError:
        return 0xFC00 if v < 0 else 0x7C00


def fp16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def quantize_group_scalar(vals) -> tuple[float, int, list[int]]:
    """One group (any length): returns (f32 scale, zero, codes).

    Weight quantization › How it works / Code: widen [min, max] to contain 0,
    scale = (max-min)/15, zero = round(-min/scale) clamped, code = clamp(round(w/scale)+zero).
    """
    vals = [float(v) for v in vals]
    for v in vals:
        if not math.isfinite(v):
            raise ValueError("non-finite weight")
        if f32(v) != v:
            raise ValueError("weights must be binary32 values")
    lo = min(min(vals), 0.0)
    hi = max(max(vals), 0.0)
    if hi > lo:
        s = f32(ieee_div(f32(hi - lo), float(QMAX)))
    else:
        s = 1.0
    zc = clamp_code(round_away(f32(ieee_div(-lo, s))))   # f32 zero, used by the codes
    z = to_code(zc)                                       # stored byte
    codes = []
    for w in vals:
        t = f32(ieee_div(w, s))
        codes.append(to_code(f32(round_away(t) + zc)))
    return s, z, codes


def quantize_scalar(w_rows, group: int = GROUP):
    """Row-wise scalar quantizer.  Returns (packed rows as bytes, scale16 bits, zeros)."""
    packed, s16, zs = [], [], []
    for row in w_rows:
        row = [float(v) for v in row]
        if len(row) % group or len(row) % 2:
            raise ValueError("row length must be a multiple of the group size")
        codes_row, s_row, z_row = [], [], []
        for g0 in range(0, len(row), group):
            s, z, codes = quantize_group_scalar(row[g0:g0 + group])
            codes_row += codes
            s_row.append(fp16_bits(s))
            z_row.append(z)
        # two codes per byte, even index in the low nibble
        b = bytes(codes_row[2 * j] | (codes_row[2 * j + 1] << 4) for j in range(len(row) // 2))
        packed.append(b)
        s16.append(s_row)
        zs.append(z_row)
    return packed, s16, zs


def dot_scalar(packed_row: bytes, s16_row, z_row, x, group: int = GROUP) -> float:
    """sum_k w_hat[k] * x[k] with w_hat = (code - zero) * scale16, correctly rounded sum."""
    terms = []
    for k, xv in enumerate(x):
        b = packed_row[k // 2]
        q = (b >> 4) if (k & 1) else (b & 0x0F)
        g = k // group
        terms.append((int(q) - int(z_row[g])) * fp16_value(int(s16_row[g])) * float(xv))
    return math.fsum(terms)


def dot_factored_exact(packed_row: bytes, s16_row, z_row, x, group: int = GROUP) -> Fraction:
    """Weight quantization › How it works: per group scale*(sum q*x - zero*sum x), in exact rationals."""
    acc = Fraction(0)
    for g in range(len(x) // group):
        qx = Fraction(0)
        sx = Fraction(0)
        for k in range(g * group, (g + 1) * group):
            b = packed_row[k // 2]
            q = (b >> 4) if (k & 1) else (b & 0x0F)
            qx += int(q) * Fraction(float(x[k]))
            sx += Fraction(float(x[k]))
        acc += Fraction(fp16_value(int(s16_row[g]))) * (qx - int(z_row[g]) * sx)
    return acc


# ---------------------------------------------------------------------------
# Vectorised path: NumPy float32 ufuncs (each is one IEEE binary32 operation)
# ---------------------------------------------------------------------------

def _round_away_np(t: np.ndarray) -> np.ndarray:
    t64 = t.astype(np.float64)
    return np.copysign(np.floor(np.abs(t64) + 0.5), t64)


def _to_code_np(t: np.ndarray) -> np.ndarray:
    c = np.clip(t, 0.0, float(QMAX))
    c = np.where(np.isnan(c), 0.0, c)
    return c.astype(np.uint8)


def quantize_ref(w: np.ndarray, group: int = GROUP):
    """Quantize W [N, K] (binary32) group-wise along K.

    Returns (packed uint8 [N, K/2], scales float16 [N, K/group], zeros uint8 [N, K/group]).
    Weight quantization › How it works / Code, step by step on whole arrays.
    """
    packed, s, z = quantize_ref_f32(w, group)
    return packed, s.astype(np.float16), z


def quantize_ref_f32(w: np.ndarray, group: int = GROUP):
    """``quantize_ref`` with the binary32 scale returned unrounded (the stored formats
    round it to fp16 or bf16)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("W must be 2-D [N, K]")
    n, k = w.shape
    if k % group or group % 2:
        raise ValueError("K must be a multiple of the group size")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    g = w.reshape(n, k // group, group)
    f0 = np.float32(0.0)
    lo = np.minimum(g.min(axis=2), f0)
    hi = np.maximum(g.max(axis=2), f0)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
        span = (hi - lo).astype(np.float32)
        s = np.where(hi > lo, span / np.float32(QMAX), np.float32(1.0)).astype(np.float32)
        zc = np.clip(_round_away_np((-lo) / s), 0.0, float(QMAX)).astype(np.float32)  # NaN kept
        z = _to_code_np(zc)
        t = g / s[:, :, None]
        codes = _to_code_np(_round_away_np(t).astype(np.float32) + zc[:, :, None])
    codes = codes.reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, s, z


# ---------------------------------------------------------------------------
# Symmetric variant (page "Quantization" › "How it really works" › "The mechanics: scale,
# round, clamp"; page "LLM Quantization Architecture in Depth" › "Number formats, scales
# and granularity"): one step per group of 128, step = max|w| / 7 (1 for an all-zero
# group), code = clamp(round(w / step), -8, 7) with halves to even (the rounding of both
# pages' examples), one binary32 operation per step.  It is stored in the method's own
# format as code + 8 with zero 8, so w_hat = (stored - zero) * scale16 is unchanged.
# ---------------------------------------------------------------------------
SYM_ZERO = 8
SYM_TOP = 7


def quantize_symmetric_ref(w: np.ndarray, group: int = GROUP):
    """Symmetric 4-bit quantization of W [N, K] (binary32) in the canonical arrays.

    Returns (packed uint8 [N, K/2], scales float16 [N, K/group], zeros uint8 [N, K/group],
    all zeros 8).  A quotient that is NaN (a step that underflows to 0 on 0/0) clamps to
    -8, and +-inf clamp to the ends, as the C fmin/fmax clamp does.
    """
    packed, s, z = quantize_symmetric_ref_f32(w, group)
    return packed, s.astype(np.float16), z


def quantize_symmetric_ref_f32(w: np.ndarray, group: int = GROUP):
    """``quantize_symmetric_ref`` with the binary32 step returned unrounded."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("W must be 2-D [N, K]")
    n, k = w.shape
    if k % group or group % 2:
        raise ValueError("K must be a multiple of the group size")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    g = w.reshape(n, k // group, group)
    amax = np.abs(g).max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore", under="ignore"):
        s = np.where(amax > 0, amax / np.float32(SYM_TOP), np.float32(1.0)).astype(np.float32)
        t = g / s[:, :, None]
        q = np.fmin(np.fmax(np.rint(t), np.float32(-SYM_TOP - 1)), np.float32(SYM_TOP))
    codes = (q.astype(np.int16) + SYM_ZERO).astype(np.uint8).reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    zeros = np.full((n, k // group), SYM_ZERO, dtype=np.uint8)
    return packed, s, zeros


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Codes [N, K] from packed bytes [N, K/2]: low nibble = even index."""
    packed = np.asarray(packed, dtype=np.uint8)
    n, kh = packed.shape
    q = np.empty((n, 2 * kh), dtype=np.uint8)
    q[:, 0::2] = packed & 0x0F
    q[:, 1::2] = packed >> 4
    return q


def dequant_ref(packed, scales16, zeros, group: int = GROUP, rows=None) -> np.ndarray:
    """w_hat = (q - zero) * scale16 in fp64 (exact), optionally for a subset of rows."""
    packed = np.asarray(packed)
    scales16 = np.asarray(scales16)
    zeros = np.asarray(zeros)
    if rows is not None:
        packed, scales16, zeros = packed[rows], scales16[rows], zeros[rows]
    q = unpack_codes(packed).astype(np.float64)
    n, k = q.shape
    qg = q.reshape(n, k // group, group)
    s = scales16.astype(np.float64)[:, :, None]
    z = zeros.astype(np.float64)[:, :, None]
    return ((qg - z) * s).reshape(n, k)


def gemv_ref(packed, scales16, zeros, x, group: int = GROUP, rows=None, chunk: int = 2048):
    """y [M, N] = x @ w_hat.T in fp64 (dequantize, then dot), row chunks to bound memory."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    idx = np.arange(np.asarray(packed).shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((x.shape[0], idx.size), dtype=np.float64)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        wh = dequant_ref(packed, scales16, zeros, group, rows=sel)
        out[:, c0:c0 + sel.size] = x @ wh.T
    return out


def gemv_factored_ref(packed, scales16, zeros, x, group: int = GROUP):
    """The factored per-group form: sum_g scale16 * (sum q*x - zero * sum x), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    q = unpack_codes(packed).astype(np.float64)
    n, k = q.shape
    kg = k // group
    qg = q.reshape(n, kg, group)
    xg = x.reshape(x.shape[0], kg, group)
    qx = np.einsum("ngk,mgk->mng", qg, xg)
    sx = xg.sum(axis=2)  # [M, kg]
    s = np.asarray(scales16).astype(np.float64)
    z = np.asarray(zeros).astype(np.float64)
    return (s[None] * (qx - z[None] * sx[:, None, :])).sum(axis=2)


def tolerance_ref(packed, scales16, zeros, x, group: int = GROUP, rows=None,
                  rel: float = 1e-3, chunk: int = 2048):
    """Per-output bound rel * sum_k |w_hat[n, k] * x[m, k]|."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    if x.ndim == 1:
        x = x[None, :]
    idx = np.arange(np.asarray(packed).shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((x.shape[0], idx.size), dtype=np.float64)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        wh = np.abs(dequant_ref(packed, scales16, zeros, group, rows=sel))
        out[:, c0:c0 + sel.size] = x @ wh.T
    return rel * out


def bits_per_weight(n_weights: int, packed_len: int, n_scales: int, n_zeros: int,
                    scale_bits: int = 16, zero_bits: int = 8) -> float:
    """Storage bits per weight of a quantized tensor."""
    return (packed_len * 8 + n_scales * scale_bits + n_zeros * zero_bits) / n_weights
