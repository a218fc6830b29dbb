"""Pins for the CPU oracle, against things the oracle does not compute itself.

Each test fixes part of the oracle to a definition outside it: exact rational
arithmetic with an independent binary32 rounding, the IEEE binary16 encoding,
brute-force searches over tiny groups, hand-derived cases from the page
"Weight quantization" (sections "How it works" and "Code"), the page's own
error assertion, closed-form sizes and invariants.
"""

import math
import os
import random
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import quant_error

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# Independent exact helpers (not used by the oracle)
# ---------------------------------------------------------------------------

def exact_f32(q: Fraction) -> float:
    """Nearest binary32 to the rational q, ties to even mantissa, found by exact comparison."""
    c = np.float32(float(q))
    if not np.isfinite(c):
        return float(c)
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        if not np.isfinite(cand):
            continue
        d = abs(Fraction(float(cand)) - q)
        even = (int(np.array(cand, dtype=np.float32).view(np.uint32)) & 1) == 0
        if best is None or d < best[0] or (d == best[0] and even):
            best = (d, cand)
    return float(best[1])


def brute_round_away(t: Fraction) -> int:
    """Integer nearest to t; at an exact half pick the one farther from zero (search, no formula)."""
    base = math.floor(t)
    cands = [base - 1, base, base + 1, base + 2]
    dist = [abs(Fraction(c) - t) for c in cands]
    m = min(dist)
    tied = [c for c, d in zip(cands, dist) if d == m]
    return max(tied, key=abs)


def brute_code(t_plus_z: Fraction, sign_t: int) -> int:
    """Code in [0, 15] nearest to t+z; at a tie step away from zero of t."""
    cands = list(range(16))
    dist = [abs(Fraction(c) - t_plus_z) for c in cands]
    m = min(dist)
    tied = [c for c, d in zip(cands, dist) if d == m]
    if len(tied) == 1:
        return tied[0]
    return max(tied) if sign_t > 0 else min(tied)


def reference_group(vals, G=None):
    """The page's group quantizer worked with exact rationals and exact_f32 rounding."""
    lo = min(min(vals), 0.0)
    hi = max(max(vals), 0.0)
    if hi > lo:
        span = exact_f32(Fraction(hi) - Fraction(lo))
        s = exact_f32(Fraction(span) / 15)
    else:
        s = 1.0
    assert s > 0, "test grid avoids scale underflow"
    zq = exact_f32(Fraction(-lo) / Fraction(s))
    z = min(max(brute_round_away(Fraction(zq)), 0), 15)
    codes = []
    for w in vals:
        t = exact_f32(Fraction(w) / Fraction(s))
        r = brute_round_away(Fraction(t))
        codes.append(min(max(r + z, 0), 15))
    return s, z, codes


# ---------------------------------------------------------------------------
# binary32 / binary16 emulation
# ---------------------------------------------------------------------------

def test_f32_rounding_matches_exact_definition():
    rng = random.Random(5)
    for _ in range(3000):
        a = float(np.float32(rng.uniform(-1e3, 1e3)))
        b = float(np.float32(rng.choice([rng.uniform(-10, 10), 15.0, 7.0, 3.0])))
        if b == 0:
            continue
        ex = exact_f32(Fraction(a) / Fraction(b))
        assert oracle.f32(a / b) == ex                       # scalar path (fp64 then round)
        assert float(np.float32(a) / np.float32(b)) == ex    # vectorised path (float32 ufunc)


def test_f32_subnormal_and_overflow():
    tiny = 2.0 ** -149
    assert oracle.f32(tiny) == tiny
    assert oracle.f32(tiny * 0.5) == 0.0           # tie to even (0)
    assert oracle.f32(tiny * 1.5) == 2 * tiny      # tie to even (2)
    assert oracle.f32(3.5e38) == math.inf


def _golden_binary16():
    rows = []
    with open(os.path.join(GOLDEN, "binary16_values.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            v, b = [t.strip() for t in line.split("|")]
            rows.append((float(eval(v, {"__builtins__": {}})), int(b, 16)))
    return rows


@pytest.mark.parametrize("value,bits", _golden_binary16())
def test_binary16_encoding(value, bits):
    assert oracle.fp16_bits(value) == bits
    arr = np.array([value], dtype=np.float32)
    with np.errstate(over="ignore"):
        assert int(arr.astype(np.float16).view(np.uint16)[0]) == bits


def test_round_away_brute_force():
    ts = [k / 2 for k in range(-40, 41)] + [0.49999997, -0.49999997, 2.5000002, 1e7 + 0.5]
    rng = random.Random(1)
    ts += [float(np.float32(rng.uniform(-20, 20))) for _ in range(500)]
    for t in ts:
        t32 = float(np.float32(t))
        assert oracle.round_away(t32) == brute_round_away(Fraction(t32))
    # the f32 trap the reading avoids: 0.49999997 + 0.5 rounds to 1 in f32
    assert oracle.round_away(0.4999999701976776) == 0.0


# ---------------------------------------------------------------------------
# Quantizer
# ---------------------------------------------------------------------------

def _golden_cases():
    out = []
    with open(os.path.join(GOLDEN, "page_formula_cases.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            name, w, s16, z, codes = [t.strip() for t in line.split("|")]
            out.append((name, [float(np.float32(v)) for v in w.split()], int(s16, 16), int(z),
                        [int(c) for c in codes.split()]))
    return out


@pytest.mark.parametrize("name,w,s16,z,codes", _golden_cases())
def test_hand_derived_groups(name, w, s16, z, codes):
    s, zz, cc = oracle.quantize_group_scalar(w)
    assert oracle.fp16_bits(s) == s16 and zz == z and cc == codes, name
    # vectorised path on the same group (padded to a 128-wide row by repetition)
    reps = 128 // len(w)
    row = np.array(w * reps, dtype=np.float32)[None, :]
    p, sv, zv = oracle.quantize_ref(row)
    q = oracle.unpack_codes(p)[0]
    assert list(q[: len(w)]) == codes
    assert int(sv.view(np.uint16)[0, 0]) == s16 and int(zv[0, 0]) == z


def _grid():
    sub = 2.0 ** -149
    return [0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 1.5, -2.5, 2.5, 3.0, -6.5, 8.5, 7.5, -7.5, 0.1, -0.3,
            1e-3, -2e-3, 0.75, -0.05, 37.0, -11.0, 1e-30, sub * 1000, -sub * 3000]


def test_brute_force_groups_of_two():
    g = _grid()
    for a in g:
        for b in g:
            vals = [float(np.float32(a)), float(np.float32(b))]
            lo, hi = min(min(vals), 0.0), max(max(vals), 0.0)
            if hi > lo and exact_f32(Fraction(exact_f32(Fraction(hi) - Fraction(lo))) / 15) == 0:
                continue
            s, z, codes = oracle.quantize_group_scalar(vals)
            rs, rz, rc = reference_group(vals)
            assert (s, z, codes) == (rs, rz, rc), vals


def test_brute_force_groups_of_four_and_code_search():
    rng = random.Random(7)
    g = _grid()
    for _ in range(3000):
        vals = [float(np.float32(rng.choice(g) * rng.choice([1, 1, 0.37, 3.1]))) for _ in range(4)]
        s, z, codes = oracle.quantize_group_scalar(vals)
        rs, rz, rc = reference_group(vals)
        assert (s, z, codes) == (rs, rz, rc), vals
        # codes are the nearest codes to f32(w/s) + zero, ties away from zero of w/s
        for w, c in zip(vals, codes):
            t = Fraction(exact_f32(Fraction(w) / Fraction(s)))
            assert c == brute_code(t + z, 1 if t > 0 else -1)


def test_scalar_and_vectorised_quantizers_agree_on_single_layer_rows():
    w, _ = synth.page_single_layer(16, 4096)
    p, s16, z = oracle.quantize_ref(w)
    P, S, Z = oracle.quantize_scalar(w.tolist())
    for i in range(w.shape[0]):
        assert bytes(p[i]) == P[i]
    assert np.array_equal(s16.view(np.uint16), np.array(S, dtype=np.uint16))
    assert np.array_equal(z, np.array(Z, dtype=np.uint8))


def _groups_stats(w):
    p, s16, z = oracle.quantize_ref(w)
    q = oracle.unpack_codes(p).astype(np.int64)
    n, k = w.shape
    kg = k // 128
    # f32 scale recomputed the page's way (only for the bound below)
    g = w.reshape(n, kg, 128).astype(np.float64)
    lo = np.minimum(g.min(axis=2), 0.0)
    hi = np.maximum(g.max(axis=2), 0.0)
    s = np.where(hi > lo, (np.float32(hi - lo) / np.float32(15)).astype(np.float64), 1.0)
    return p, s16, z, q.reshape(n, kg, 128), g, s


@pytest.mark.parametrize("kind", ["uniform", "normal_outliers", "skewed"])
def test_reconstruction_error_at_most_half_step(kind):
    rng = np.random.default_rng(3)
    if kind == "uniform":
        w = (0.02 * rng.uniform(-1, 1, (64, 1024))).astype(np.float32)
    elif kind == "normal_outliers":
        w = (0.02 * rng.standard_normal((64, 1024))).astype(np.float32)
        w[:, rng.choice(1024, 10, replace=False)] *= 20
    else:
        w = (0.02 * rng.standard_normal((64, 1024)) + 0.03).astype(np.float32)
    p, s16, z, q, g, s = _groups_stats(w)
    assert q.min() >= 0 and q.max() <= 15 and z.max() <= 15
    deq = (q - z[:, :, None]) * s[:, :, None]
    err = np.abs(deq - g)
    assert np.all(err <= s[:, :, None] * (0.5 + 1e-5))
    s16v = s16.astype(np.float64)[:, :, None]
    deq16 = (q - z[:, :, None]) * s16v
    assert np.all(np.abs(deq16 - g) <= s[:, :, None] * (0.5 + 1e-5) + 15 * np.abs(s[:, :, None] - s16v))
    # every non-empty group uses an end of the code range (|q - z| >= 7 somewhere)
    assert np.all(np.abs(q - z[:, :, None]).max(axis=2) >= 7)


def test_zero_is_exactly_representable():
    rng = np.random.default_rng(11)
    w = (0.02 * rng.standard_normal((32, 1024))).astype(np.float32)
    w[:, ::37] = 0.0
    p, s16, z = oracle.quantize_ref(w)
    q = oracle.unpack_codes(p)
    wh = oracle.dequant_ref(p, s16, z)
    zero_pos = w == 0.0
    assert np.all(q[zero_pos] == np.repeat(z, 128, axis=1)[zero_pos])
    assert np.all(wh[zero_pos] == 0.0)


def test_nibble_order_even_index_low():
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 0] = -1.0          # code 0 after widening (zero = 15 when the group is non-positive)
    w[0, 1] = 0.0           # code 15
    p, s16, z = oracle.quantize_ref(w)
    assert int(z[0, 0]) == 15
    assert int(p[0, 0]) == (0 | (15 << 4))


def test_scale_underflow_corner_follows_f32_semantics():
    sub = 2.0 ** -149
    # widened range of 3 subnormal steps: f32 scale underflows to 0
    vals = [-3 * sub, sub, 0.0, 2 * sub]
    s, z, codes = oracle.quantize_group_scalar(vals)
    assert s == 0.0 and z == 15
    # w/0 -> -inf (code 0), +inf (code 15), NaN (code 0)
    assert codes == [0, 15, 0, 15]
    # lo = 0: -lo/0 is NaN, the f32 zero stays NaN and every code becomes 0
    s, z, codes = oracle.quantize_group_scalar([sub, 2 * sub, 0.0, sub])
    assert s == 0.0 and z == 0 and codes == [0, 0, 0, 0]
    row = np.array([[-3 * sub, sub, 0.0, 2 * sub] * 32, [sub, 2 * sub, 0.0, sub] * 32], dtype=np.float32)
    p, s16, zz = oracle.quantize_ref(row)
    q = oracle.unpack_codes(p)
    assert list(q[0, :4]) == [0, 15, 0, 15] and list(q[1, :4]) == [0, 0, 0, 0]
    assert list(zz[:, 0]) == [15, 0] and list(s16.view(np.uint16)[:, 0]) == [0, 0]


def test_nonfinite_rejected():
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 5] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize_ref(w)
    with pytest.raises(ValueError):
        oracle.quantize_group_scalar([0.0, math.inf])


# ---------------------------------------------------------------------------
# Dot product / GEMV
# ---------------------------------------------------------------------------

def _small_problem(seed=0, n=6, k=384, m=3):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    p, s16, z = oracle.quantize_ref(w)
    return w, x, p, s16, z


def test_factored_identity_exact():
    w, x, p, s16, z = _small_problem()
    for n in range(p.shape[0]):
        for m in range(x.shape[0]):
            exact = Fraction(0)
            wh = oracle.dequant_ref(p, s16, z, rows=[n])[0]
            for k in range(x.shape[1]):
                exact += Fraction(float(wh[k])) * Fraction(float(x[m, k]))
            fac = oracle.dot_factored_exact(bytes(p[n]), list(s16.view(np.uint16)[n]), list(z[n]), x[m])
            assert fac == exact
            assert abs(oracle.dot_scalar(bytes(p[n]), list(s16.view(np.uint16)[n]), list(z[n]), x[m])
                       - float(exact)) <= 1e-15 * max(1.0, abs(float(exact)))


def test_gemv_ref_matches_exact_and_factored():
    w, x, p, s16, z = _small_problem(1, n=16, k=1024, m=4)
    y = oracle.gemv_ref(p, s16, z, x)
    yf = oracle.gemv_factored_ref(p, s16, z, x)
    bound = oracle.tolerance_ref(p, s16, z, x)
    for n in range(16):
        for m in range(4):
            exact = float(oracle.dot_factored_exact(bytes(p[n]), list(s16.view(np.uint16)[n]), list(z[n]), x[m]))
            scale = bound[m, n] / 1e-3
            assert abs(y[m, n] - exact) <= 1e-12 * scale
            assert abs(yf[m, n] - exact) <= 1e-12 * scale


def test_one_hot_returns_dequantized_column():
    w, x, p, s16, z = _small_problem(2, n=8, k=256, m=1)
    wh = oracle.dequant_ref(p, s16, z)
    for k in (0, 1, 127, 128, 255):
        e = np.zeros((1, 256), dtype=np.float32)
        e[0, k] = 1.0
        y = oracle.gemv_ref(p, s16, z, e)
        assert np.array_equal(y[0], wh[:, k])


def test_page_error_assertion_on_its_own_draws():
    # the page's program: w = 0.02*U(-1,1) for 4096 draws, then x = 4096 more draws
    r = synth.xorshift_uniform(8192)
    w = (np.float32(0.02) * r[:4096])[None, :]
    x = r[4096:][None, :]
    p, s16, z = oracle.quantize_ref(w)
    y = oracle.gemv_ref(p, s16, z, x)[0, 0]
    exact = float(np.sum(w[0].astype(np.float64) * x[0].astype(np.float64)))
    scale = float(np.sum(np.abs(w[0].astype(np.float64) * x[0])))
    assert abs(y - exact) < 0.02 * scale


def test_page_error_assertion_on_single_layer_rows():
    w, x = synth.page_single_layer(4096, 4096)
    rows = np.arange(0, 4096, 97)
    p, s16, z = oracle.quantize_ref(w[rows])
    y = oracle.gemv_ref(p, s16, z, x)[0]
    exact = w[rows].astype(np.float64) @ x[0].astype(np.float64)
    scale = np.abs(w[rows].astype(np.float64)) @ np.abs(x[0].astype(np.float64))
    assert np.all(np.abs(y - exact) < 0.02 * scale)


# ---------------------------------------------------------------------------
# Sizes and workload arithmetic
# ---------------------------------------------------------------------------

def test_bits_per_weight_closed_forms():
    w = np.zeros((1, 4096), dtype=np.float32)
    p, s16, z = oracle.quantize_ref(w)
    # the page's formula: packed bytes * 8 + 16-bit scales + 4-bit zeros
    assert oracle.bits_per_weight(4096, p.size, s16.size, z.size, 16, 4) == 4.15625
    # the stored format here: fp16 scale and a byte zero per 128
    assert oracle.bits_per_weight(4096, p.size, s16.size, z.size, 16, 8) == 4.1875
    # fp16 scale alone: 4 + 16/128
    assert oracle.bits_per_weight(4096, p.size, s16.size, 0, 16, 0) == 4.125


def test_seventy_b_layer_arithmetic():
    per_layer = sum(n * k for n, k in synth.LLAMA70B_SHAPES.values())
    assert 80 * per_layer == 68_451_041_280            # "roughly 68.5 billion" linear weights
    bytes_per_layer = sum(n * k // 2 + (n * k // 128) * 3 for n, k in synth.LLAMA70B_SHAPES.values())
    assert 80 * bytes_per_layer == 35_829_841_920      # "about 36 GB"


# ---------------------------------------------------------------------------
# Input generator (the page's xorshift stream)
# ---------------------------------------------------------------------------

def test_xorshift_stream_against_definition():
    s = synth.XORSHIFT_SEED
    mask = (1 << 64) - 1
    states = synth.xorshift_states(5000)
    r = synth.xorshift_uniform(5000)
    for i in range(5000):
        s ^= (s << 13) & mask
        s ^= s >> 7
        s ^= (s << 17) & mask
        assert int(states[i]) == s
        if i % 97 == 0:
            u = exact_f32(Fraction(s >> 11))
            u = exact_f32(Fraction(u) / Fraction(2 ** 53))
            u = exact_f32(Fraction(u) * 2)
            u = exact_f32(Fraction(u) - 1)
            assert float(r[i]) == u


def test_regression_snapshot_of_single_layer():
    """Oracle outputs on the 4096x4096 page workload, stored by tests/golden/make_golden.py."""
    path = os.path.join(GOLDEN, "single_layer_snapshot.txt")
    snap = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            key, val = line.split("=", 1)
            snap[key.strip()] = val.strip()
    w, x = synth.page_single_layer(4096, 4096)
    rows = [int(v) for v in snap["rows"].split()]
    p, s16, z = oracle.quantize_ref(w[rows])
    y = oracle.gemv_ref(p, s16, z, x)[0]
    for i, r in enumerate(rows):
        assert bytes(p[i][:32]).hex() == snap[f"packed_head_{r}"]
        assert " ".join(f"{v:04x}" for v in s16.view(np.uint16)[i][:8]) == snap[f"s16_head_{r}"]
        assert " ".join(str(v) for v in z[i][:8]) == snap[f"zero_head_{r}"]
        assert float.fromhex(snap[f"y_{r}"]) == y[i]


# ---------------------------------------------------------------------------
# Error harness: page "Quantization", section "Code" (its printed table) and
# "Try it", item 1 (asymmetric scales per group of 128)
# ---------------------------------------------------------------------------

def _page_error_table():
    rows = []
    with open(os.path.join(GOLDEN, "page_error_table.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([f.strip() for f in line.split("|")])
    return rows


def test_error_harness_reproduces_page_table():
    """Every printed figure of the page's table, at the page's precision."""
    got = quant_error.table(synth.page_error_matrix())
    want = _page_error_table()
    assert [g[0] for g in got] == [r[0] for r in want]
    for (name, bits, db, rel, gb, ms), r in zip(got, want):
        assert [f"{bits:.2f}", f"{db:.1f}", f"{100 * rel:.2f}", f"{gb:.0f}", f"{ms:.1f}"] == r[1:], name


def _e4m3_values():
    """All finite E4M3 values >= 0 from the bit fields (4 exponent, 3 mantissa, bias 7)."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue   # the NaN code
            vals.append((m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(sorted(vals))


def test_e4m3_rounding_is_nearest_value_ties_to_even():
    grid = _e4m3_values()
    assert grid[-1] == 448.0 and grid[1] == 2.0 ** -9
    rng = np.random.default_rng(3)
    t = np.concatenate([rng.uniform(0, 460, 4000), 2.0 ** rng.uniform(-12, 8, 4000),
                        (grid[:-1] + grid[1:]) / 2, grid])
    got = quant_error.e4m3_round(t)
    for v, r in zip(t, got):
        a = min(v, 448.0)
        d = np.abs(grid - a)
        idx = np.flatnonzero(d == d.min())
        # a tie goes to the even mantissa field; in the sorted grid each binade holds the
        # fields 0..7 in order, so the field's parity is the index's parity
        if len(idx) == 2:
            idx = [i for i in idx if i % 2 == 0]
        assert r == grid[idx[0]], v
    assert np.array_equal(quant_error.e4m3_round(-t), -got)


def test_asymmetric_g128_step_and_error_against_symmetric():
    """Try it, item 1.  The page prints no answer, so the value itself is unpinned; what is
    fixed: with the range widened to hold 0, hi - lo <= 2 max|w|, so the asymmetric step
    (hi - lo) / 15 is at most 14/15 of the symmetric step max|w| / 7 in every group, and
    the reconstruction error must beat the symmetric group-128 row of the table."""
    w = synth.page_error_matrix()
    w32, w_hat, packed, s16, zeros = quant_error.asym_w4(w)
    g = w32.astype(np.float64).reshape(w.shape[0], -1, 128)
    sym_step = np.abs(g).max(axis=2) / 7
    asym_step = s16.view(np.float16).astype(np.float64)
    assert np.all(asym_step <= sym_step * (14 / 15) * (1 + 2.0 ** -10))
    db, rel = quant_error.sqnr_db(w32.astype(np.float64), w_hat)
    sym_db = [r[2] for r in quant_error.table(w) if r[0] == "INT4 group 128"][0]
    assert db > sym_db + 0.5
    assert 0.09 < rel < 0.1224


# ---------------------------------------------------------------------------
# Symmetric variant: page "Quantization" › "How it really works" (scale, round, clamp),
# stored as code + 8 with zero 8
# ---------------------------------------------------------------------------

def brute_round_even(t: Fraction) -> int:
    """Integer nearest to t; at an exact half the even one (search, no formula)."""
    base = math.floor(t)
    cands = [base - 1, base, base + 1, base + 2]
    dist = [abs(Fraction(c) - t) for c in cands]
    m = min(dist)
    tied = [c for c, d in zip(cands, dist) if d == m]
    return [c for c in tied if c % 2 == 0][0] if len(tied) > 1 else tied[0]


def reference_symmetric_group(vals):
    amax = max(abs(v) for v in vals)
    s = exact_f32(Fraction(amax) / 7) if amax > 0 else 1.0
    assert s > 0, "test grid avoids step underflow"
    codes = []
    for v in vals:
        t = exact_f32(Fraction(v) / Fraction(s))
        codes.append(min(max(brute_round_even(Fraction(t)), -8), 7) + 8)
    return s, codes


def _sym_check(rows):
    w = np.array(rows, dtype=np.float32)
    g = w.shape[1]
    p, s16, z = oracle.quantize_symmetric_ref(w, group=g)
    codes = oracle.unpack_codes(p)
    assert np.all(z == 8)
    for i, row in enumerate(rows):
        s, want = reference_symmetric_group([float(np.float32(v)) for v in row])
        assert list(codes[i]) == want, (row, list(codes[i]), want)
        with np.errstate(over="ignore"):   # steps beyond binary16 range round to inf on both sides
            assert s16[i, 0] == np.float16(s)


def test_symmetric_brute_force_pairs_and_quads_with_ties():
    grid = [0.0, 3.5, -3.5, 2.5, -0.5, 0.5, 7.0, -7.0, 1.5, 6.5, -6.5, 1e-30, 2.0 ** -140, 0.1]
    _sym_check([[a, b] for a in grid for b in grid])
    rng = np.random.default_rng(9)
    quads = []
    for _ in range(2000):
        kind = rng.integers(3)
        if kind == 0:      # multiples of 1/2 with the largest magnitude 7: exact half ties
            v = rng.integers(-14, 15, 4) / 2.0
            v[rng.integers(4)] = 7.0 * rng.choice([-1, 1])
        elif kind == 1:
            v = rng.standard_normal(4) * 10.0 ** rng.uniform(-30, 30)
        else:
            v = np.round(rng.standard_normal(4) * 8) / 8
        quads.append([float(np.float32(x)) for x in v])
    _sym_check(quads)


def test_symmetric_invariants_and_page_table_row():
    rng = np.random.default_rng(10)
    w = (0.02 * rng.standard_normal((64, 1024))).astype(np.float32)
    w[3, 5] = 0.7
    w[7, :128] = 0.0
    p, s16, z = oracle.quantize_symmetric_ref(w)
    codes = oracle.unpack_codes(p).astype(np.int64)
    g = w.astype(np.float64).reshape(64, 8, 128)
    amax = np.abs(g).max(axis=2)
    s32 = np.where(amax > 0, (amax.astype(np.float32) / np.float32(7)).astype(np.float64), 1.0)
    q = codes.reshape(64, 8, 128) - 8
    assert q.min() >= -7 and q.max() <= 7            # |w / step| <= 7: the clamp never acts
    assert np.all(np.abs(q * s32[:, :, None] - g) <= s32[:, :, None] / 2 * (1 + 1e-6))
    assert np.all(codes[w == 0.0] == 8)               # zero stays exactly representable
    top = np.abs(g) == amax[:, :, None]
    assert np.all(np.abs(q[top & (amax[:, :, None] > 0)]) == 7)
    # the page's symmetric group-128 row on its own matrix, with the stored binary16 step
    wp = synth.page_error_matrix()
    p, s16, z = oracle.quantize_symmetric_ref(wp.astype(np.float32))
    db, rel = quant_error.sqnr_db(wp, oracle.dequant_ref(p, s16, z))
    row = [r for r in _page_error_table() if r[0] == "INT4 group 128"][0]
    assert [f"{db:.1f}", f"{100 * rel:.2f}"] == row[2:4]

