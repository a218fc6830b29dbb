"""Pins of the oracle's tolerance functions (CPU only).

Every GPU parity verdict compares |y_gpu - y_ref| with the oracle's per-output bound
1e-3 * sum_k |w_hat[n, k] * x[m, k]|.  These tests recompute that sum from the stored
bytes with exact rationals -- decoding codes, scales and zeros here from the format's
definition, not through the oracle's own dequantization -- and require the oracle's
bounds to agree to fp64 rounding.  The inputs mix signs so that a dropped absolute value
changes the sum, and a wrong relative factor changes every bound.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle

REL = Fraction(1, 1000)


def _pack(q: np.ndarray) -> np.ndarray:
    """Codes [N, K] -> bytes [N, K/2], the even index in the low nibble."""
    q = q.astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def _f16(bits: int) -> Fraction:
    """Exact value of a binary16 bit pattern (finite)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    return sign * Fraction(1024 + m, 1 << 10) * Fraction(2) ** (e - 15)


def _bf16(bits: int) -> Fraction:
    """Exact value of a bfloat16 bit pattern (finite)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 1 << 7) * Fraction(2) ** -126
    return sign * Fraction(128 + m, 1 << 7) * Fraction(2) ** (e - 127)


def _exact_bound(codes, zeros, scales, x, group):
    """1e-3 * sum_k |(q - zero) * scale * x| in rationals; zeros/scales per group (lists)."""
    n, k = codes.shape
    out = np.empty((x.shape[0], n), dtype=object)
    for m in range(x.shape[0]):
        xs = [Fraction(float(v)) for v in x[m]]
        for r in range(n):
            tot = Fraction(0)
            for c in range(k):
                g = c // group
                tot += abs((int(codes[r, c]) - int(zeros[r][g])) * scales[r][g] * xs[c])
            out[m, r] = REL * tot
    return out


def _assert_close(got, exact):
    for (m, r), e in np.ndenumerate(exact):
        g = Fraction(float(got[m, r]))
        assert abs(g - e) <= abs(e) * Fraction(1, 10**12), (m, r, float(got[m, r]), float(e))


def _random_case(rng, n, k, group):
    codes = rng.integers(0, 16, (n, k))
    zeros = rng.integers(0, 16, (n, k // group))
    s16 = rng.uniform(1e-3, 0.1, (n, k // group)).astype(np.float16)
    x = rng.standard_normal((3, k)).astype(np.float32)
    return codes, zeros, s16, x


def test_tolerance_ref_hand_case():
    # one group of 128: codes 7, 1, 5 at inputs 0..2 (zero 5, scale 0.5), x = 2, 3, 0.5
    # w_hat = 1, -2, 0 -> sum |w_hat x| = |1*2| + |-2*3| + 0 = 8 (the signed sum is -4)
    q = np.full((1, 128), 5)
    q[0, :3] = (7, 1, 5)
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :3] = (2.0, 3.0, 0.5)
    b = oracle.tolerance_ref(_pack(q), np.array([[0.5]], dtype=np.float16),
                             np.array([[5]], dtype=np.uint8), x)
    assert b.shape == (1, 1) and b[0, 0] == 8e-3


@pytest.mark.parametrize("seed", [1, 2])
def test_tolerance_ref_against_exact_sum(seed):
    rng = np.random.default_rng(seed)
    codes, zeros, s16, x = _random_case(rng, 5, 256, 128)
    got = oracle.tolerance_ref(_pack(codes), s16, zeros.astype(np.uint8), x)
    scales = [[_f16(int(b)) for b in row] for row in s16.view(np.uint16)]
    _assert_close(got, _exact_bound(codes, zeros.tolist(), scales, x, 128))
    # and a subset of rows
    got_rows = oracle.tolerance_ref(_pack(codes), s16, zeros.astype(np.uint8), x, rows=[4, 1])
    full = _exact_bound(codes, zeros.tolist(), scales, x, 128)
    _assert_close(got_rows, full[:, [4, 1]])


FORMATS = [oracle.Format(g, sb, zb, sym) for g in (32, 128) for sb in (False, True)
           for zb in (4, 8) for sym in (False, True)]


@pytest.mark.parametrize("fmt", FORMATS, ids=str)
def test_tolerance_format_ref_against_exact_sum(fmt):
    rng = np.random.default_rng(fmt.group + 2 * fmt.zero_bits + int(fmt.scale_bf16) + 7 * int(fmt.symmetric))
    n, k = 3, 128
    codes = rng.integers(0, 16, (n, k))
    kg = k // fmt.group
    zeros = np.full((n, kg), 8) if fmt.symmetric else rng.integers(0, 16, (n, kg))
    vals = rng.uniform(1e-3, 0.1, (n, kg)).astype(np.float32)
    if fmt.scale_bf16:
        bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
        scales = [[_bf16(int(b)) for b in row] for row in bits]
    else:
        bits = vals.astype(np.float16).view(np.uint16)
        scales = [[_f16(int(b)) for b in row] for row in bits]
    if fmt.zero_bits == 8:
        zstored = zeros.astype(np.uint8)
    else:
        flat = zeros.reshape(-1)
        if flat.size % 2:
            flat = np.r_[flat, 0]
        zstored = (flat[0::2] | (flat[1::2] << 4)).astype(np.uint8)
    x = rng.standard_normal((2, k)).astype(np.float32)
    got = oracle.tolerance_format_ref(_pack(codes), bits, zstored, x, fmt)
    _assert_close(got, _exact_bound(codes, zeros.tolist(), scales, x, fmt.group))


def test_tolerance_int8_ref_against_exact_sum():
    rng = np.random.default_rng(3)
    cx = rng.integers(-128, 128, (2, 64)).astype(np.int8)
    cw = rng.integers(-128, 128, (3, 64)).astype(np.int8)
    sx = rng.uniform(1e-3, 1.0, 2).astype(np.float32)
    sw = rng.uniform(1e-3, 1.0, 3).astype(np.float32)
    got = oracle.tolerance_int8_ref(cx, sx, cw, sw)
    exact = np.empty((2, 3), dtype=object)
    for m in range(2):
        for n in range(3):
            exact[m, n] = REL * sum(abs(int(cx[m, k]) * Fraction(float(sx[m])) * int(cw[n, k]) *
                                        Fraction(float(sw[n]))) for k in range(64))
    _assert_close(got, exact)


def _e4m3(b: int) -> Fraction:
    """Exact value of an OCP E4M3 byte (finite): sign, 4 exponent bits (bias 7), 3 mantissa."""
    sign = -1 if b & 0x80 else 1
    e = (b >> 3) & 0xF
    m = b & 7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(2) ** -6
    return sign * Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


def test_tolerance_fp8_ref_against_exact_sum():
    rng = np.random.default_rng(4)
    finite = [b for b in range(256) if (b & 0x7F) != 0x7F]
    cx = rng.choice(finite, (2, 64)).astype(np.uint8)
    cw = rng.choice(finite, (3, 64)).astype(np.uint8)
    sx = rng.uniform(1e-3, 1.0, 2).astype(np.float32)
    sw = rng.uniform(1e-3, 1.0, 3).astype(np.float32)
    got = oracle.tolerance_fp8_ref(cx, sx, cw, sw)
    exact = np.empty((2, 3), dtype=object)
    for m in range(2):
        for n in range(3):
            exact[m, n] = REL * sum(abs(_e4m3(int(cx[m, k])) * Fraction(float(sx[m])) *
                                        _e4m3(int(cw[n, k])) * Fraction(float(sw[n]))) for k in range(64))
    _assert_close(got, exact)
