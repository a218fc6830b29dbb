"""Pins of the INT8 W8A8 oracle against definitions outside it: the page's printed INT8
per-channel error row, a brute-force nearest-integer search with ties to even in exact
rationals, hand-worked rows, and exact rationals for the product."""

from fractions import Fraction

import numpy as np

import oracle
import synth
from oracle import quant_error


def test_page_int8_per_channel_row_of_error_table():
    # page "Quantization" › "Code": INT8 per-channel gives 38.2 dB and 1.22 %
    w = synth.page_error_matrix()
    c, s = oracle.quantize_rows_int8_ref(w)
    sqnr, rel = quant_error.sqnr_db(w.astype(np.float64), oracle.dequant_int8_ref(c, s))
    assert f"{sqnr:.1f}" == "38.2" and f"{100 * rel:.2f}" == "1.22"


def test_codes_are_the_nearest_integer_with_ties_to_even():
    rng = np.random.default_rng(13)
    a = rng.standard_normal((40, 64)) * np.exp(rng.uniform(-5, 5, (40, 1)))
    # rows built to hit exact ties: max 127 (step 1) and values at k + 1/2
    a[0] = np.concatenate([[127.0], np.arange(-31.5, 31.5, 1.0)])
    a[1] = 0.0
    c, s = oracle.quantize_rows_int8_ref(a)
    for r in range(a.shape[0]):
        amax = Fraction(float(np.max(np.abs(a[r]))))
        step = Fraction(float(amax / 127)) if amax else Fraction(1)
        for k in range(a.shape[1]):
            t = Fraction(float(a[r, k])) / step
            lo = t.numerator // t.denominator
            frac = t - lo
            want = lo + 1 if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2) else lo
            want = max(-128, min(127, want))
            assert c[r, k] == want, (r, k, float(t))
    assert list(c[0, :4]) == [127, -32, -30, -30]   # -31.5 -> -32, -30.5 -> -30, -29.5 -> -30
    assert np.all(c[1] == 0) and s[1] == 1.0
    assert np.all(np.abs(c[2:]).max(axis=1) == 127)


def test_gemm_ref_against_exact_rationals():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((3, 64)).astype(np.float32)
    w = (0.02 * rng.standard_normal((4, 64))).astype(np.float32)
    cx, sx = oracle.quantize_rows_int8_ref(x)
    cw, sw = oracle.quantize_rows_int8_ref(w)
    y = oracle.gemm_int8_ref(cx, sx, cw, sw)
    for m in range(3):
        for n in range(4):
            exact = (sum(int(cx[m, k]) * int(cw[n, k]) for k in range(64))
                     * Fraction(float(sx[m])) * Fraction(float(sw[n])))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)
