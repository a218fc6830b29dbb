"""CPU oracle for W8A8 in INT8: per-row symmetric 8-bit codes and their product.

TEST INFRASTRUCTURE ONLY, under the same rules as ``w4_oracle``: only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may import
it; the product path never does, and it shares no code with the HIP library.

What it computes (page "Quantization", sections "How it really works" › "The
mechanics: scale, round, clamp" and "Code": symmetric INT8 with one absmax
scale per block, per-tensor or per-channel; page "LLM Quantization Architecture
in Depth" › "Why fewer bits make decoding faster": W8A8 in INT8 or FP8 speeds up
prefill; › "Number formats, scales and granularity": dynamic per-token scales
for activations):

* one block per row (an output channel of W, a token of X);
* step = max |row| / 127 (1 if that is 0); code = round(value / step), halves to
  even (Python's ``round`` in the page's program), clamped to [-128, 127];
* Y[m, n] = sum_k x_hat[m, k] * w_hat[n, k] in fp64 with x_hat = code * step.

Readings where the pages are silent (each pinned by a test): the step and the
quotient are fp64 as in the page's Python program; the stored step is that fp64
step rounded to binary32, and the product uses the stored step.
"""

from __future__ import annotations

import numpy as np

INT8_MAX = 127


def quantize_rows_int8_ref(a: np.ndarray):
    """Per-row symmetric INT8 codes [R, K] int8 and binary32 steps [R]."""
    a = np.asarray(a, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input")
    amax = np.max(np.abs(a), axis=1)
    s = amax / INT8_MAX
    s = np.where(s == 0.0, 1.0, s)
    q = np.clip(np.rint(a / s[:, None]), -INT8_MAX - 1, INT8_MAX)
    return q.astype(np.int8), s.astype(np.float32)


def dequant_int8_ref(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[:, None]


def gemm_int8_ref(cx, sx, cw, sw) -> np.ndarray:
    """Y = x_hat w_hat^T in fp64."""
    return dequant_int8_ref(cx, sx) @ dequant_int8_ref(cw, sw).T


def tolerance_int8_ref(cx, sx, cw, sw, rel: float = 1e-3) -> np.ndarray:
    return rel * (np.abs(dequant_int8_ref(cx, sx)) @ np.abs(dequant_int8_ref(cw, sw)).T)
