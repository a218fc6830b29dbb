"""Pins of the format-variant oracle (group 32/64/128, bf16 or fp16 scales, 8- or 4-bit
zeros, symmetric or asymmetric) against definitions outside it: hand-worked bit patterns,
torch's CPU bfloat16 conversion, a brute-force nearest search in exact rationals, the
scalar emulation of the quantizer, and the error bounds of rounding to a grid."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import Format

FORMATS = [Format(g, sb, zb, sym) for g in (32, 64, 128) for sb in (False, True)
           for zb in (8, 4) for sym in (False, True)]


def test_bf16_bits_hand_values():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -23,
                     -2.0, 2.0 ** -149, 0.0, -0.0, 3.0e38], dtype=np.float32)
    # 1 + 2^-8 is halfway between 0x3F80 and 0x3F81 (even kept); 1 + 3*2^-8 halfway between
    # 0x3F81 and 0x3F82 (even kept); just above the first tie rounds up; the smallest
    # subnormal rounds to +0; 3e38 stays finite (0x7F62 = 3.0e38 rounded)
    got = oracle.bf16_bits(vals)
    assert list(got[:8]) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x0000, 0x0000, 0x8000]
    assert oracle.bf16_value(got[8]) == pytest.approx(3.0e38, rel=2 ** -8)
    assert list(oracle.bf16_value(np.array([0x3F80, 0xC000, 0x3E80], dtype=np.uint16))) == [1.0, -2.0, 0.25]


def test_bf16_bits_match_torch_cpu_conversion():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(200_000).astype(np.float32) * np.float32(0.01)
    # exact ties: the low 16 bits 0x8000 with both parities of the kept half
    u = v.view(np.uint32)
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000
    v = u.view(np.float32)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_bits(v), ref)


def test_bf16_bits_are_the_nearest_value_brute_force():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(300) * 10.0 ** rng.integers(-6, 6, 300)).astype(np.float32)
    for x, b in zip(v, oracle.bf16_bits(v)):
        t = int(np.float32(x).view(np.uint32)) >> 16
        cands = [t, t + 1]
        vals = [Fraction(float(oracle.bf16_value(np.uint16(c)))) for c in cands]
        d = [abs(Fraction(float(x)) - c) for c in vals]
        best = cands[0] if d[0] < d[1] else cands[1] if d[1] < d[0] else (t if t % 2 == 0 else t + 1)
        assert int(b) == best


def test_zero_nibbles_hand_example_and_round_trip():
    assert list(oracle.pack_zero_nibbles(np.array([[3, 12, 7]]))) == [0xC3, 0x07]
    rng = np.random.default_rng(5)
    for n, kg in ((1, 1), (3, 5), (7, 64), (4, 2)):
        z = rng.integers(0, 16, (n, kg)).astype(np.uint8)
        zp = oracle.pack_zero_nibbles(z)
        assert zp.size == (n * kg + 1) // 2
        assert np.array_equal(oracle.unpack_zero_nibbles(zp, n, kg), z)
    with pytest.raises(ValueError):
        oracle.pack_zero_nibbles(np.array([16]))


@pytest.mark.parametrize("group", [32, 64])
def test_small_groups_match_the_scalar_emulation(group):
    rng = np.random.default_rng(group)
    w = (0.02 * rng.standard_normal((6, 256))).astype(np.float32)
    w[0, :group] = 0.0            # an empty range
    w[1, :group] = np.abs(w[1, :group])   # one sign only
    packed, s16, z = oracle.quantize_ref(w, group)
    sp, ss, sz = oracle.quantize_scalar(w.tolist(), group)
    assert [bytes(r) for r in packed] == sp
    assert s16.view(np.uint16).tolist() == ss
    assert z.tolist() == sz


@pytest.mark.parametrize("fmt", FORMATS, ids=str)
def test_format_codes_and_error_bounds(fmt):
    rng = np.random.default_rng(fmt.group + 2 * fmt.scale_bf16 + fmt.zero_bits + fmt.symmetric)
    n, k = 9, 384
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[2, : fmt.group] = 0.0
    packed, sbits, zeros = oracle.quantize_format_ref(w, fmt)
    # codes are those of the base quantizer at the same group size
    base = oracle.quantize_symmetric_ref if fmt.symmetric else oracle.quantize_ref
    bp, bs, bz = base(w, fmt.group)
    assert np.array_equal(packed, bp)
    z = oracle.zeros_u8(zeros, n, k, fmt)
    assert np.array_equal(z, bz)
    if fmt.zero_bits == 4:
        assert zeros.size == oracle.zero_bytes(n, k, fmt) == (n * (k // fmt.group) + 1) // 2
    # the stored scale is the f32 step rounded to the stored type
    s32 = (oracle.quantize_symmetric_ref_f32 if fmt.symmetric else oracle.quantize_ref_f32)(w, fmt.group)[1]
    sv = oracle.scale_value(sbits, fmt.scale_bf16)
    rel = 2.0 ** -8 if fmt.scale_bf16 else 2.0 ** -11   # half an ulp: 8 or 11 significant bits
    assert np.all(np.abs(sv - s32) <= rel * np.abs(s32.astype(np.float64)))
    # |w_hat - w| <= step/2 + 15 |step - stored| (+ the symmetric clamp of the extreme code:
    # the largest magnitude maps to +-7 or -8 exactly, so the bound holds there too)
    wh = oracle.dequant_format_ref(packed, sbits, zeros, fmt)
    sg = np.repeat(s32.astype(np.float64), fmt.group, axis=1)
    svg = np.repeat(sv, fmt.group, axis=1)
    bound = sg / 2 + 15 * np.abs(sg - svg) + 1e-12 * sg
    assert np.all(np.abs(wh - w.astype(np.float64)) <= bound)
    # dequantization is exact: (q - z) has 5 bits, the stored scale 11 or 8
    q = oracle.unpack_codes(packed)
    for (r, c) in ((0, 0), (4, 131), (8, k - 1)):
        g = c // fmt.group
        exact = (Fraction(int(q[r, c])) - int(z[r, g])) * Fraction(float(sv[r, g]))
        assert Fraction(float(wh[r, c])) == exact


def test_format_gemv_one_hot_and_rows():
    fmt = Format(32, True, 4, False)
    rng = np.random.default_rng(9)
    w = (0.02 * rng.standard_normal((5, 256))).astype(np.float32)
    p, s, z = oracle.quantize_format_ref(w, fmt)
    wh = oracle.dequant_format_ref(p, s, z, fmt)
    x = np.zeros((2, 256))
    x[0, 7] = 1.0
    x[1, 200] = 1.0
    y = oracle.gemv_format_ref(p, s, z, x, fmt)
    assert np.array_equal(y[0], wh[:, 7]) and np.array_equal(y[1], wh[:, 200])
    assert np.array_equal(oracle.gemv_format_ref(p, s, z, x, fmt, rows=[1, 3]), y[:, [1, 3]])


def test_canonical_format_is_the_base_quantizer():
    rng = np.random.default_rng(10)
    w = (0.02 * rng.standard_normal((4, 256))).astype(np.float32)
    p, s, z = oracle.quantize_ref(w)
    fp, fs, fz = oracle.quantize_format_ref(w, oracle.CANONICAL)
    assert np.array_equal(p, fp) and np.array_equal(s.view(np.uint16), fs) and np.array_equal(z, fz)


def test_format_bits_per_weight():
    # page "Weight quantization" › "Code": the bits of 4096 weights with fp16 scales and
    # 4-bit zeros, (2048*8 + 32*16 + 32*4) / 4096; "Complexity and constants": about 4.16
    fmt = Format(128, False, 4, False)
    assert oracle.format_bits_per_weight(fmt) == (2048 * 8 + 32 * 16 + 32 * 4) / 4096 == 4.15625
    assert oracle.format_bits_per_weight(Format()) == 4.1875
    assert oracle.format_bits_per_weight(Format(32, True, 8, False)) == 4.75
    for f in FORMATS:
        n, k = 6, 1024
        assert oracle.format_bytes(n, k, f) * 8 == oracle.format_bits_per_weight(f) * n * k
