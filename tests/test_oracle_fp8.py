"""Pins of the FP8 (E4M3) W8A8 oracle against definitions outside it: hand-decoded bytes,
torch's CPU float8_e4m3fn type (decode and nearest-even conversion), the page's printed
error table, exact rationals for the product, and the rounding bound of the grid."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import quant_error


def test_decode_hand_values():
    d = oracle.e4m3_decode
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6 and d(0x3F) == 1.875 and d(0x40) == 2.0
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.E4M3_VALUES
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    assert np.array_equal(got[~both_nan], ref[~both_nan])
    pos = got[:0x7F]
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0


def test_rounding_matches_torch_nearest_even_conversion():
    rng = np.random.default_rng(5)
    t = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 20000) * 2.0 ** -5,
                        rng.standard_normal(20000) * 20])
    # exact midpoints between neighbouring values, both parities
    pos = oracle.E4M3_VALUES[1:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    t = np.concatenate([t, mids, -mids, pos, -pos]).astype(np.float32).astype(np.float64)
    t = t[np.abs(t) <= 448]
    ref = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = quant_error.e4m3_round(t)
    assert np.array_equal(got, ref)
    # and the encoded byte is the byte torch stores
    ref_bytes = torch.from_numpy(t.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nz = got != 0
    assert np.array_equal(oracle.e4m3_encode(got)[nz], ref_bytes[nz])


def test_encode_round_trip_and_signed_zero():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.E4M3_VALUES[codes]
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    # a negative quotient that rounds to zero keeps its sign; an exact zero is +0
    c, s = oracle.quantize_rows_fp8_ref(np.array([[1.0, -1e-9, 0.0, -0.0]]))
    assert list(c[0]) == [0x7E, 0x80, 0x00, 0x00]
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([1.0625]))


def test_row_quantization_invariants():
    rng = np.random.default_rng(7)
    a = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1)))).astype(np.float32)
    a[3] = 0.0
    a[4] = 0.0
    a[4, 17] = -3.5
    codes, scales = oracle.quantize_rows_fp8_ref(a)
    amax = np.abs(a.astype(np.float64)).max(axis=1)
    s64 = np.where(amax == 0, 1.0, amax / 448.0)
    assert np.array_equal(scales, s64.astype(np.float32))
    q = oracle.E4M3_VALUES[codes]
    # the largest magnitude of every non-zero row lands on +-448
    nz = amax > 0
    assert np.all(np.abs(q[nz]).max(axis=1) == 448.0)
    assert np.all(codes[3] == 0) and scales[3] == 1.0
    assert codes[4, 17] == 0xFE and np.count_nonzero(codes[4] & 0x7F) == 1
    # within half a grid step of the quotient (grid of 3 mantissa bits, floor 2^-9)
    t = a / s64[:, None]
    step = 2.0 ** (np.maximum(np.floor(np.log2(np.maximum(np.abs(t), 1e-300))), -6) - 3)
    assert np.all(np.abs(q - t) <= step / 2 + 1e-12 * np.abs(t))


def test_page_fp8_per_channel_row_of_error_table():
    # page "Quantization" › "Code": FP8 E4M3 per-channel gives 31.7 dB and 2.61 %
    w = synth.page_error_matrix()
    codes, scales = oracle.quantize_rows_fp8_ref(w)
    w_hat = oracle.dequant_fp8_ref(codes, scales)
    sqnr, rel = quant_error.sqnr_db(w.astype(np.float64), w_hat)
    assert f"{sqnr:.1f}" == "31.7" and f"{100 * rel:.2f}" == "2.61"


def test_gemm_ref_against_exact_rationals():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    w = (0.02 * rng.standard_normal((5, 64))).astype(np.float32)
    cx, sx = oracle.quantize_rows_fp8_ref(x)
    cw, sw = oracle.quantize_rows_fp8_ref(w)
    y = oracle.gemm_fp8_ref(cx, sx, cw, sw)
    for m in range(3):
        for n in range(5):
            exact = sum(Fraction(oracle.E4M3_VALUES[cx[m, k]]) * Fraction(oracle.E4M3_VALUES[cw[n, k]])
                        for k in range(64)) * Fraction(float(sx[m])) * Fraction(float(sw[n]))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)
    tol = oracle.tolerance_fp8_ref(cx, sx, cw, sw)
    assert np.all(tol >= 1e-3 * np.abs(y) - 1e-18)
