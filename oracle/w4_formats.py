"""CPU oracle for the storage variants of the 4-bit weight format.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the product path never
calls it and shares no code with it.

A format is (group, scale type, zero width, symmetric):

* group: 32, 64 or 128 consecutive weights along K share one scale and zero (page
  "Quantization" › "Code": the error table compares int4 groups of 128 and of 32;
  page "Weight quantization" › "How it works": groups along the input dimension);
* scale type: the f32 step is stored as binary16 (round to nearest even; page
  "Weight quantization" › "Code": fp16 scales on disk) or as bfloat16 (round to
  nearest even of the binary32 value; page "Weight quantization" › "Implementation
  notes": scales in fp16 or bf16);
* zero width: one byte per group, or two groups per byte (page "Weight
  quantization" › "Code" and "Complexity and constants": a 4-bit zero per group).
  The nibbles are packed over the row-major [N, K/group] array read as one flat
  sequence, the even index in the low nibble, as the codes are;
* symmetric: the step max|w|/7 with halves to even and zero 8, as
  ``quantize_symmetric_ref``; otherwise the asymmetric method of ``quantize_ref``.

The codes and the f32 step of every group are exactly those of ``quantize_ref`` /
``quantize_symmetric_ref`` at the same group size (only the stored scale differs), so
w_hat = (code - zero) * stored_scale and y = x @ w_hat^T in fp64 as before.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import w4_oracle as _o


@dataclass(frozen=True)
class Format:
    group: int = 128
    scale_bf16: bool = False
    zero_bits: int = 8
    symmetric: bool = False

    def check(self, k: int) -> None:
        if self.group not in (32, 64, 128):
            raise ValueError("group must be 32, 64 or 128")
        if self.zero_bits not in (4, 8):
            raise ValueError("zero_bits must be 4 or 8")
        if k % self.group:
            raise ValueError("K must be a multiple of the group size")


CANONICAL = Format()


def bf16_bits(v) -> np.ndarray:
    """bfloat16 bit patterns of binary32 values: round to nearest, ties to even, on the
    binary32 bit pattern (the 16 dropped bits decide; a tie keeps the even upper half)."""
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    upper = u >> 16
    lower = u & 0xFFFF
    up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    return (upper + up.astype(np.uint64)).astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """Values (fp64) of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def scale_value(scale_bits, scale_bf16: bool) -> np.ndarray:
    """Values (fp64) of stored scales given as 16-bit patterns."""
    b = np.asarray(scale_bits, dtype=np.uint16)
    if scale_bf16:
        return bf16_value(b)
    return b.view(np.float16).astype(np.float64)


def pack_zero_nibbles(zeros: np.ndarray) -> np.ndarray:
    """[N, Kg] zeros (0..15) -> ceil(N*Kg/2) bytes: flat index i at byte i//2, low nibble
    for even i."""
    z = np.asarray(zeros, dtype=np.uint8).reshape(-1)
    if np.any(z > 15):
        raise ValueError("a zero does not fit in 4 bits")
    if z.size % 2:
        z = np.concatenate([z, np.zeros(1, dtype=np.uint8)])
    return (z[0::2] | (z[1::2] << 4)).astype(np.uint8)


def unpack_zero_nibbles(zp: np.ndarray, n: int, kg: int) -> np.ndarray:
    """Inverse of ``pack_zero_nibbles`` for an [n, kg] array."""
    zp = np.asarray(zp, dtype=np.uint8).reshape(-1)
    flat = np.empty(2 * zp.size, dtype=np.uint8)
    flat[0::2] = zp & 0x0F
    flat[1::2] = zp >> 4
    return flat[: n * kg].reshape(n, kg)


def zero_bytes(n: int, k: int, fmt: Format) -> int:
    kg = k // fmt.group
    return n * kg if fmt.zero_bits == 8 else (n * kg + 1) // 2


def quantize_format_ref(w: np.ndarray, fmt: Format):
    """Quantize W [N, K] (binary32) in format ``fmt``.

    Returns (packed uint8 [N, K/2], scale bits uint16 [N, Kg], zeros): zeros are uint8
    [N, Kg] for 8-bit zeros, or the packed nibbles (``pack_zero_nibbles``) for 4-bit ones.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    fmt.check(w.shape[1])
    if fmt.symmetric:
        packed, s32, z = _o.quantize_symmetric_ref_f32(w, fmt.group)
    else:
        packed, s32, z = _o.quantize_ref_f32(w, fmt.group)
    if fmt.scale_bf16:
        sbits = bf16_bits(s32)
    else:
        sbits = s32.astype(np.float16).view(np.uint16)
    zeros = pack_zero_nibbles(z) if fmt.zero_bits == 4 else z
    return packed, sbits, zeros


def zeros_u8(zeros, n: int, k: int, fmt: Format) -> np.ndarray:
    """The [N, Kg] zero bytes of a format's zero array."""
    if fmt.zero_bits == 4:
        return unpack_zero_nibbles(zeros, n, k // fmt.group)
    return np.asarray(zeros, dtype=np.uint8).reshape(n, k // fmt.group)


def dequant_format_ref(packed, scale_bits, zeros, fmt: Format, rows=None) -> np.ndarray:
    """w_hat = (q - zero) * stored scale, in fp64 (exact), optionally for a subset of rows."""
    packed = np.asarray(packed)
    n, kh = packed.shape
    k = 2 * kh
    z = zeros_u8(zeros, n, k, fmt)
    s = scale_value(scale_bits, fmt.scale_bf16).reshape(n, k // fmt.group)
    if rows is not None:
        packed, s, z = packed[rows], s[rows], z[rows]
    q = _o.unpack_codes(packed).astype(np.float64)
    nr = q.shape[0]
    qg = q.reshape(nr, k // fmt.group, fmt.group)
    return ((qg - z.astype(np.float64)[:, :, None]) * s[:, :, None]).reshape(nr, k)


def gemv_format_ref(packed, scale_bits, zeros, x, fmt: Format, rows=None, chunk: int = 2048):
    """y [M, N] = x @ w_hat.T in fp64 (dequantize, then dot)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim == 1:
        x = x[None, :]
    n = np.asarray(packed).shape[0]
    idx = np.arange(n) if rows is None else np.asarray(rows)
    out = np.empty((x.shape[0], idx.size), dtype=np.float64)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        out[:, c0:c0 + sel.size] = x @ dequant_format_ref(packed, scale_bits, zeros, fmt, sel).T
    return out


def tolerance_format_ref(packed, scale_bits, zeros, x, fmt: Format, rows=None,
                         rel: float = 1e-3, chunk: int = 2048):
    """Per-output bound rel * sum_k |w_hat[n, k] * x[m, k]|."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    if x.ndim == 1:
        x = x[None, :]
    n = np.asarray(packed).shape[0]
    idx = np.arange(n) if rows is None else np.asarray(rows)
    out = np.empty((x.shape[0], idx.size), dtype=np.float64)
    for c0 in range(0, idx.size, chunk):
        sel = idx[c0:c0 + chunk]
        out[:, c0:c0 + sel.size] = x @ np.abs(dequant_format_ref(packed, scale_bits, zeros, fmt, sel)).T
    return rel * out


def format_bits_per_weight(fmt: Format) -> float:
    """Storage bits per weight: 4 for the code, plus the scale and zero of each group."""
    return 4.0 + (16 + fmt.zero_bits) / fmt.group


def format_bytes(n: int, k: int, fmt: Format) -> int:
    """Bytes of the stored tensor: codes, scales, zeros."""
    return n * k // 2 + 2 * n * (k // fmt.group) + zero_bytes(n, k, fmt)
