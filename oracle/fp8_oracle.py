"""CPU oracle for W8A8 in FP8 E4M3: per-row scaled E4M3 codes and their product.

TEST INFRASTRUCTURE ONLY, under the same rules as ``w4_oracle``: only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may import
it; the product path never does, and it shares no code with the HIP library.

What it computes:

* E4M3 (page "Quantization", section "Floating point: FP8" and its program in
  "Code"; page "LLM Quantization Architecture in Depth" › "Number formats,
  scales and granularity"): a sign, 4 exponent bits and 3 mantissa bits, largest
  value 448, subnormals below 2^-6.  A value is rounded to it by capping its
  magnitude at 448 and rounding, halves to even, on the grid of 3 mantissa bits
  of its binary exponent (exponents below -6 use the grid of -6); that rounding
  is ``quant_error.e4m3_round``, which reproduces the page's printed table.
* a block's scale is its largest magnitude over 448 (1 if that is 0), the
  per-tensor / per-channel rule of the page's program; here a block is one row:
  one output channel of W, and one token of X (page "LLM Quantization
  Architecture in Depth": activations take dynamic per-token scales; W8A8 in
  FP8 is the format that makes prefill faster, section "Why fewer bits make
  decoding faster").
* Y[m, n] = sum_k x_hat[m, k] * w_hat[n, k] in fp64, x_hat = value(code) *
  scale, the same for w (dequantize, then multiply).

Readings where the pages are silent (each pinned by a test):

* the scale and the quotient value / scale are fp64, as in the page's Python
  program, so the codes are those the page's arithmetic gives; the stored
  scale is that fp64 scale rounded to binary32, and the product uses the stored
  scale;
* codes are stored in the OCP E4M3 bit layout (sign, exponent with bias 7,
  mantissa; 0x7E is 448; 0x7F and 0xFF are NaN and never produced); a value that
  rounds to zero keeps the sign of its quotient (code 0x80 for a negative one),
  an exact zero is code 0x00.
"""

from __future__ import annotations

import math

import numpy as np

from .quant_error import e4m3_round

FP8_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of an E4M3 byte: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9          # subnormal: m/8 * 2^-6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# value of every byte (NaN at 0x7F and 0xFF)
E4M3_VALUES = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)

# the 127 non-negative finite values in code order (codes 0x00 .. 0x7E), increasing
_POS = E4M3_VALUES[:0x7F]


def e4m3_encode(q: np.ndarray) -> np.ndarray:
    """Codes of values that lie on the E4M3 grid (|q| <= 448); the sign bit follows the
    sign of q, so -0.0 gives 0x80."""
    q = np.asarray(q, dtype=np.float64)
    mag = np.abs(q)
    idx = np.searchsorted(_POS, mag)
    if np.any(idx >= _POS.size) or not np.array_equal(_POS[np.minimum(idx, _POS.size - 1)], mag):
        raise ValueError("value not on the E4M3 grid")
    return (idx.astype(np.uint8) | np.where(np.signbit(q), 0x80, 0).astype(np.uint8)).astype(np.uint8)


def quantize_rows_fp8_ref(a: np.ndarray):
    """Per-row E4M3 quantization of a [R, K] array (binary32 or bfloat16 values).

    Returns (codes uint8 [R, K], scales float32 [R])."""
    a = np.asarray(a, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input")
    amax = np.max(np.abs(a), axis=1)
    s = amax / FP8_MAX
    s = np.where(s == 0.0, 1.0, s)
    t = a / s[:, None]
    q = e4m3_round(t)
    # e4m3_round gives +0.0 for an exact zero and keeps the quotient's sign otherwise
    return e4m3_encode(q), s.astype(np.float32)


def dequant_fp8_ref(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """value(code) * stored scale, fp64."""
    return E4M3_VALUES[np.asarray(codes)] * np.asarray(scales, dtype=np.float64)[:, None]


def gemm_fp8_ref(cx, sx, cw, sw) -> np.ndarray:
    """Y = x_hat w_hat^T in fp64 (x_hat [M, K], w_hat [N, K])."""
    return dequant_fp8_ref(cx, sx) @ dequant_fp8_ref(cw, sw).T


def tolerance_fp8_ref(cx, sx, cw, sw, rel: float = 1e-3) -> np.ndarray:
    """rel * sum_k |x_hat[m, k] w_hat[n, k]| per output."""
    return rel * (np.abs(dequant_fp8_ref(cx, sx)) @ np.abs(dequant_fp8_ref(cw, sw)).T)
