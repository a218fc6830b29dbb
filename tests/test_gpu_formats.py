"""GPU parity of the format variants (group 32/64/128, bf16 or fp16 scales, 8- or 4-bit
zeros, symmetric or asymmetric): quantization bit-exact against the oracle, the prepared
layout round trip, and w4_gemv_fmt within the tolerance of the method."""

import numpy as np
import pytest
import torch

import dequant_gemv_w4_amd as w4
import oracle
import synth
from _util import assert_within, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

FORMATS = [oracle.Format(g, sb, zb, sym) for g in (32, 64, 128) for sb in (False, True)
           for zb in (8, 4) for sym in (False, True)]


def _wf(fmt):
    return w4.W4Format.make(fmt.group, fmt.scale_bf16, fmt.zero_bits, fmt.symmetric)


def _scale_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _edge_matrix(n, k, seed):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[0] = 0.0                                   # empty ranges
    w[1, :64] = np.abs(w[1, :64])                # one sign only
    w[2, 32:96] = -np.abs(w[2, 32:96])
    w[3, :128] = np.float32(3.0)                 # constant groups
    w[4] = np.round(w[4] / 0.002) * np.float32(0.001)   # many exact halves of the step
    w[5, :32] = 1e-30                            # tiny but non-zero
    return w


def _gpu_quant(W, fmt):
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    p, s, z = w4.w4_quantize_fmt(W, _wf(fmt), status=status)
    torch.cuda.synchronize()
    return p, s, z, int(status.item())


@pytest.mark.parametrize("fmt", FORMATS, ids=str)
@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_quantize_formats_bit_exact(fmt, wdtype):
    n, k = 37, 384      # 37 * 384 / group groups: odd for group 128 (zero nibble tail)
    w = _edge_matrix(n, k, fmt.group + fmt.zero_bits)
    W = torch.from_numpy(w).to(DEV)
    if wdtype == "bf16":
        W = W.to(torch.bfloat16)
        w = to_np32(W)
    p, s, z, st = _gpu_quant(W, fmt)
    rp, rs, rz = oracle.quantize_format_ref(w, fmt)
    assert np.array_equal(p.cpu().numpy(), rp), "packed"
    assert np.array_equal(_scale_bits(s), rs), "scale bits"
    assert np.array_equal(z.cpu().numpy().reshape(-1), np.asarray(rz).reshape(-1)), "zeros"
    # W4_STATUS_SCALE_ZERO exactly when a group with a non-zero weight stores a zero scale
    # (the 1e-30 group at group 32 with binary16 scales)
    nonzero = np.any(w.reshape(n, k // fmt.group, fmt.group) != 0, axis=2)
    expect = 4 if np.any(nonzero & ((rs & 0x7FFF) == 0)) else 0
    assert st == expect


@pytest.mark.parametrize("fmt", FORMATS, ids=str)
def test_prepare_round_trip(fmt):
    n, k = 37, 384
    W = torch.from_numpy(_edge_matrix(n, k, 3)).to(DEV)
    p, s, z, _ = _gpu_quant(W, fmt)
    prep = w4.w4_prepare_fmt(p, s, z, _wf(fmt))
    assert prep.numel() == w4.w4_prepared_bytes_fmt(n, k, _wf(fmt))
    p2, s2, z2 = w4.w4_unprepare_fmt(prep, n, k, _wf(fmt))
    torch.cuda.synchronize()
    assert torch.equal(p, p2) and torch.equal(s.view(torch.int16), s2.view(torch.int16))
    assert torch.equal(z, z2)


@pytest.mark.parametrize("fmt", FORMATS, ids=str)
def test_gemv_formats_against_oracle(fmt):
    n, k = 301, 1152      # ragged rows; K = 36 slices of 32 (a partial wave)
    rng = np.random.default_rng(fmt.group)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[7] = 0.0
    W = torch.from_numpy(w).to(DEV)
    p, s, z, _ = _gpu_quant(W, fmt)
    prep = w4.w4_prepare_fmt(p, s, z, _wf(fmt))
    rp, rs, rz = oracle.quantize_format_ref(w, fmt)
    x16 = torch.from_numpy(rng.standard_normal((16, k)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    x32 = torch.from_numpy(rng.standard_normal((5, k)).astype(np.float32)).to(DEV)
    worst = 0.0
    for x in [x16[:m].contiguous() for m in (1, 2, 3, 4, 5, 8, 16)] + [x32[:1].contiguous(), x32]:
        y = to_np32(w4.w4_gemv_fmt(prep, n, k, _wf(fmt), x))
        xn = to_np32(x)
        yr = oracle.gemv_format_ref(rp, rs, rz, xn, fmt)
        bound = oracle.tolerance_format_ref(rp, rs, rz, xn, fmt)
        # every row, the all-zero row 7 included: its bound is 0, so it must come out exactly 0
        r = assert_within(y, yr, bound, f"{fmt} M={x.shape[0]} {x.dtype}")
        worst = max(worst, r)
        assert np.all(y[:, 7] == 0.0)
    print(f"{fmt}: worst err/bound {worst:.3e}")


def test_gemv_format_one_hot_exact_and_bf16_output():
    fmt = oracle.Format(32, True, 4, False)
    n, k = 64, 512
    rng = np.random.default_rng(21)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    p, s, z, _ = _gpu_quant(torch.from_numpy(w).to(DEV), fmt)
    prep = w4.w4_prepare_fmt(p, s, z, _wf(fmt))
    rp, rs, rz = oracle.quantize_format_ref(w, fmt)
    wh = oracle.dequant_format_ref(rp, rs, rz, fmt)
    cols = [0, 31, 32, 200, 511]
    x = torch.zeros(len(cols), k, dtype=torch.bfloat16, device=DEV)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = to_np32(w4.w4_gemv_fmt(prep, n, k, _wf(fmt), x))
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), wh[:, c]), f"column {c}"
    # bf16 output: the f32 result rounded to nearest even
    xr = torch.from_numpy(rng.standard_normal((3, k)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    y32 = w4.w4_gemv_fmt(prep, n, k, _wf(fmt), xr)
    yb = w4.w4_gemv_fmt(prep, n, k, _wf(fmt), xr, out_dtype=torch.bfloat16)
    assert torch.equal(y32.to(torch.bfloat16), yb)


def test_canonical_layout_formats_match_w4_gemv():
    """Group 128 with binary16 scales prepares to the canonical layout: 4-bit zeros and the
    symmetric codes give the bytes of the canonical entry points, and w4_gemv_fmt takes the
    matrix-core kernels like w4_gemv does."""
    n, k = 12300, 1152
    W = synth.normal_weights(n, k, 31, DEV)
    for sym in (False, True):
        fmt = oracle.Format(128, False, 4, sym)
        p, s, z, _ = _gpu_quant(W, fmt)
        prep = w4.w4_prepare_fmt(p, s, z, _wf(fmt))
        cp, cs, cz = (w4.w4_quantize_symmetric if sym else w4.w4_quantize)(W)
        prep_c = w4.w4_prepare(cp, cs, cz)
        torch.cuda.synchronize()
        assert torch.equal(prep, prep_c)
        x = synth.normal_activations(16, k, 32, DEV)
        for m in (1, 4, 16):
            assert torch.equal(w4.w4_gemv_fmt(prep, n, k, _wf(fmt), x[:m].contiguous()),
                               w4.w4_gemv(prep_c, n, k, x[:m].contiguous()))


@pytest.mark.parametrize("fmt", [oracle.Format(32, True, 4, False), oracle.Format(64, False, 8, True)],
                         ids=str)
def test_gemv_format_70b_gate_sampled_rows(fmt):
    """A 70B gate|up-shaped matrix (57344 x 8192) in a small-group format, at M = 1 and 16:
    sampled rows (first, last and 254 random) against the oracle on the same weight rows."""
    n, k = 57344, 8192
    W = synth.normal_weights(n, k, 41, DEV)
    p, s, z, st = _gpu_quant(W, fmt)
    assert st == 0
    prep = w4.w4_prepare_fmt(p, s, z, _wf(fmt))
    rng = np.random.default_rng(42)
    rows = np.unique(np.concatenate([[0, 1, n - 1], rng.choice(n, 254, replace=False)]))
    w_rows = to_np32(W[torch.from_numpy(rows).to(DEV)])
    del W, p, s, z
    rp, rs, rz = oracle.quantize_format_ref(w_rows, fmt)
    x16 = synth.normal_activations(16, k, 43, DEV)
    for m in (1, 16):
        x = x16[:m].contiguous()
        y = to_np32(w4.w4_gemv_fmt(prep, n, k, _wf(fmt), x))[:, rows]
        xn = to_np32(x)
        r = assert_within(y, oracle.gemv_format_ref(rp, rs, rz, xn, fmt),
                          oracle.tolerance_format_ref(rp, rs, rz, xn, fmt), f"{fmt} M={m}")
        print(f"{fmt} M={m}: worst err/bound {r:.3e}")
