"""Quantization-error harness: fake-quantize a weight matrix, measure how far it moved.

TEST INFRASTRUCTURE ONLY, under the same rules as ``w4_oracle``: only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may import
it; the product path never does.

What it computes (page "Quantization", sections "How it really works" › "The
mechanics: scale, round, clamp" and "Code", whose printed run is the table this
harness must reproduce):

* the input is the page's seeded 256 x 1024 matrix with eight outliers, made
  by ``synth.page_error_matrix`` (inputs live outside the oracle);
* symmetric b-bit integer fake quantization of a block: the step is the block's
  largest magnitude divided by 2^(b-1) - 1 (1 if that is 0), values are divided
  by it, rounded to the nearest integer with halves to even (Python's
  ``round``), clamped to [-2^(b-1), 2^(b-1) - 1] and multiplied back;
* FP8 E4M3 fake quantization of a block: the block is divided by its largest
  magnitude over 448 (1 if 0); each value keeps its sign, its magnitude is
  capped at 448 and rounded (halves to even) on the grid of 3 mantissa bits of
  its binary exponent, where exponents below -6 use the subnormal grid of -6;
  the result is capped at 448 and multiplied back;
* blocks are the whole tensor, one row (per channel) or consecutive groups of
  G values along a row;
* SQNR = 10 log10(sum w^2 / sum (w - w_hat)^2) and the relative RMS error
  sqrt(sum (w - w_hat)^2 / sum w^2), both in fp64;
* the method's own asymmetric group-128 scheme (page "Weight quantization"),
  which the "Quantization" page leaves as its first exercise ("Try it", item
  1), is ``w4_oracle.quantize_ref`` followed by ``dequant_ref`` on the binary32
  weights.
"""

from __future__ import annotations

import math

import numpy as np

from . import w4_oracle


def sym_int_block(v: np.ndarray, bits: int) -> np.ndarray:
    """Symmetric round-to-nearest (halves to even) with one absmax step for the block."""
    top = 2 ** (bits - 1) - 1
    step = float(np.max(np.abs(v))) / top
    if step == 0.0:
        step = 1.0
    return np.clip(np.rint(v / step), -top - 1, top) * step


def e4m3_round(t: np.ndarray) -> np.ndarray:
    """Nearest FP8 E4M3 value (max 448, 3 mantissa bits, subnormals below 2^-6)."""
    mag = np.minimum(np.abs(t), 448.0)
    # binary exponent floor(log2 mag), exact: mag = f * 2^e with f in [0.5, 1)
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))
    exp = np.maximum(e - 1, -6)
    grid = np.ldexp(1.0, exp - 3)
    out = np.minimum(np.rint(mag / grid) * grid, 448.0)
    return np.where(t == 0, 0.0, np.copysign(out, t))


def fp8_block(v: np.ndarray) -> np.ndarray:
    """E4M3 fake quantization with one absmax-to-448 scale for the block."""
    s = float(np.max(np.abs(v))) / 448.0
    if s == 0.0:
        s = 1.0
    return e4m3_round(v / s) * s


def per_tensor(w: np.ndarray, fn) -> np.ndarray:
    return fn(w.reshape(-1)).reshape(w.shape)


def per_row(w: np.ndarray, fn) -> np.ndarray:
    return np.stack([fn(r) for r in w])


def per_group(w: np.ndarray, fn, group: int) -> np.ndarray:
    out = np.empty_like(w)
    for r in range(w.shape[0]):
        for c in range(0, w.shape[1], group):
            out[r, c:c + group] = fn(w[r, c:c + group])
    return out


def sqnr_db(w: np.ndarray, w_hat: np.ndarray) -> tuple[float, float]:
    """(SQNR in dB, relative RMS error) of w_hat against w, fp64 sums."""
    sig = float(np.sum(np.square(w)))
    err = float(np.sum(np.square(w - w_hat)))
    return 10.0 * math.log10(sig / err), math.sqrt(err / sig)


def asym_w4(w: np.ndarray, group: int = w4_oracle.GROUP):
    """The method's asymmetric 4-bit scheme on the binary32 weights.

    Returns (binary32 weights, w_hat fp64, packed, scale16 bits, zeros).
    """
    w32 = np.asarray(w, dtype=np.float32)
    packed, s16, zeros = w4_oracle.quantize_ref(w32, group=group)
    w_hat = w4_oracle.dequant_ref(packed, s16, zeros, group=group)
    return w32, w_hat, packed, s16, zeros


def asym_bits_per_weight(group: int = w4_oracle.GROUP) -> float:
    """Canonical format of the method: 4-bit codes, a 16-bit scale and a byte zero per group."""
    return 4 + (16 + 8) / group


# bits per weight in the table: codes plus one 16-bit scale per block (the page's accounting)
def page_schemes(cols: int):
    """(name, bits per weight, fake-quantizer over the whole matrix) for the page's table."""
    return [
        ("INT8 per-tensor", 8.0, lambda w: per_tensor(w, lambda v: sym_int_block(v, 8))),
        ("INT8 per-channel", 8 + 16 / cols, lambda w: per_row(w, lambda v: sym_int_block(v, 8))),
        ("FP8 E4M3 per-tensor", 8.0, lambda w: per_tensor(w, fp8_block)),
        ("FP8 E4M3 per-channel", 8 + 16 / cols, lambda w: per_row(w, fp8_block)),
        ("INT4 per-tensor", 4.0, lambda w: per_tensor(w, lambda v: sym_int_block(v, 4))),
        ("INT4 per-channel", 4 + 16 / cols, lambda w: per_row(w, lambda v: sym_int_block(v, 4))),
        ("INT4 group 128", 4 + 16 / 128, lambda w: per_group(w, lambda v: sym_int_block(v, 4), 128)),
        ("INT4 group 32", 4 + 16 / 32, lambda w: per_group(w, lambda v: sym_int_block(v, 4), 32)),
    ]


# the page sizes formats for a 70.6e9-parameter model read at 3.35 TB/s
PARAMS_70B = 70.6e9
REFERENCE_BW = 3.35e12


def model_gb(bits: float) -> float:
    return PARAMS_70B * bits / 8 / 1e9


def decode_floor_ms(bits: float) -> float:
    return model_gb(bits) * 1e9 / REFERENCE_BW * 1e3


def table(w: np.ndarray):
    """Rows (name, bits/weight, SQNR dB, rel. RMS, 70B GB, floor ms) of the page's schemes."""
    out = []
    for name, bits, fn in page_schemes(w.shape[1]):
        db, rel = sqnr_db(w, fn(w))
        out.append((name, bits, db, rel, model_gb(bits), decode_floor_ms(bits)))
    return out
