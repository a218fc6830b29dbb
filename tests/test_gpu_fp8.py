"""GPU parity of the W8A8 FP8 path (w4_fp8_quantize_rows, w4_fp8_gemm) against the oracle.

Codes and scales must match the oracle bit for bit; products must lie within
1e-3 * sum_k |x_hat[m, k] * w_hat[n, k]| of the fp64 product of the oracle's dequantized
operands.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_w4_amd as w4
import oracle
import synth
from _util import assert_within, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check_codes(codes, scales, ref_codes, ref_scales, what):
    c = codes.cpu().numpy()
    sc = scales.cpu().numpy()
    bad = np.argwhere(c != ref_codes)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[0]}: {c[tuple(bad[0])]:#x} vs {ref_codes[tuple(bad[0])]:#x}"
    assert np.array_equal(sc.view(np.uint32), ref_scales.view(np.uint32)), f"{what}: scales differ"


def test_quantize_rows_bit_exact_edge_rows():
    rng = np.random.default_rng(41)
    a = (rng.standard_normal((300, 1024)) * np.exp(rng.uniform(-20, 20, (300, 1)))).astype(np.float32)
    a[0] = 0.0                                   # all zero: scale 1, codes 0
    a[1] = 0.0
    a[1, 5] = -7.25                              # one value: -448 (0xFE)
    a[2] = rng.standard_normal(1024).astype(np.float32) * 1e-5
    a[2, 0] = 1.0                                # the rest in the subnormal range, some to -0
    a[3, :] = np.float32(3.0e38)                 # huge but finite
    a[4, ::2] = -a[4, ::2]
    A = torch.from_numpy(a).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    codes, scales = w4.w4_fp8_quantize_rows(A, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rc, rs = oracle.quantize_rows_fp8_ref(a)
    _check_codes(codes, scales, rc, rs, "f32 rows")
    assert np.count_nonzero(rc[2] == 0x80) > 0 and np.count_nonzero((rc[2] & 0x78) == 0) > 100


def test_quantize_rows_exact_and_near_midpoints():
    # rows whose largest magnitude is 448 * 2^j make the scale a power of two, so the
    # quotients are the values themselves scaled: put them on the midpoints between
    # neighbouring E4M3 values (exact ties, halves to even) and one binary32 ulp either side
    pos = oracle.E4M3_VALUES[1:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    rows = []
    for j in (-3, 0, 5):
        base = np.concatenate([mids, -mids, np.nextafter(mids, np.float32(0)),
                               np.nextafter(mids, np.float32(1000))]).astype(np.float32)
        base = np.resize(base, 1024).astype(np.float32)
        base[0] = 448.0
        rows.append((base * np.float32(2.0 ** j)).astype(np.float32))
    a = np.stack(rows)
    codes, scales = w4.w4_fp8_quantize_rows(torch.from_numpy(a).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows_fp8_ref(a)
    assert np.all(rs == np.float32(2.0) ** np.array([-3, 0, 5], dtype=np.float32))
    _check_codes(codes, scales, rc, rs, "midpoint rows")


@pytest.mark.parametrize("rows,k", [(77, 8192), (5, 128), (130, 384), (3, 8320), (2, 65536)])
def test_quantize_rows_bf16_activations(rows, k):
    X = synth.normal_activations(rows, k, 4200 + rows, DEV)
    X[:, : max(1, k // 100)] *= 20                # outlier channels
    codes, scales = w4.w4_fp8_quantize_rows(X.contiguous())
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows_fp8_ref(to_np32(X))
    _check_codes(codes, scales, rc, rs, f"bf16 {rows}x{k}")


def test_quantize_rows_nonfinite_sets_status():
    a = torch.ones(3, 256, dtype=torch.float32, device=DEV)
    a[1, 7] = float("inf")
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    w4.w4_fp8_quantize_rows(a, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 1


@pytest.mark.parametrize("m,n,k", [(200, 300, 384), (1, 1, 128), (129, 257, 1024), (64, 4096, 8192),
                                   (3, 5, 65536)])
def test_gemm_full_small(m, n, k):
    X = synth.normal_activations(m, k, 4300 + m, DEV)
    W = synth.normal_weights(n, k, 4301 + n, DEV)
    xq, sx = w4.w4_fp8_quantize_rows(X)
    wq, sw = w4.w4_fp8_quantize_rows(W)
    Y = w4.w4_fp8_gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    rcx, rsx = oracle.quantize_rows_fp8_ref(to_np32(X))
    rcw, rsw = oracle.quantize_rows_fp8_ref(to_np32(W))
    _check_codes(xq, sx, rcx, rsx, "x")
    _check_codes(wq, sw, rcw, rsw, "w")
    r = assert_within(to_np32(Y), oracle.gemm_fp8_ref(rcx, rsx, rcw, rsw),
                      oracle.tolerance_fp8_ref(rcx, rsx, rcw, rsw), f"fp8 gemm {m}x{n}x{k}")
    print(f"{m}x{n}x{k}: worst err/bound {r:.3e}")


def test_prefill_shape_sampled_outputs():
    m, n, k = 4096, 28672, 8192
    X = synth.normal_activations(m, k, 4400, DEV)
    W = synth.normal_weights(n, k, 4401, DEV)
    xq, sx = w4.w4_fp8_quantize_rows(X)
    wq, sw = w4.w4_fp8_quantize_rows(W)
    Y = w4.w4_fp8_gemm(xq, sx, wq, sw)
    Yb = w4.w4_fp8_gemm(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    Y2 = w4.w4_fp8_gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2), "not deterministic"
    rng = np.random.default_rng(43)
    rm = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 62, replace=False)]))
    rn = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 446, replace=False)]))
    x32 = to_np32(X[torch.from_numpy(rm).to(DEV)])
    w32 = to_np32(W[torch.from_numpy(rn).to(DEV)])
    del X, W
    rcx, rsx = oracle.quantize_rows_fp8_ref(x32)
    rcw, rsw = oracle.quantize_rows_fp8_ref(w32)
    _check_codes(xq[torch.from_numpy(rm).to(DEV)], sx[torch.from_numpy(rm).to(DEV)], rcx, rsx, "x rows")
    _check_codes(wq[torch.from_numpy(rn).to(DEV)], sw[torch.from_numpy(rn).to(DEV)], rcw, rsw, "w rows")
    ref = oracle.gemm_fp8_ref(rcx, rsx, rcw, rsw)
    bound = oracle.tolerance_fp8_ref(rcx, rsx, rcw, rsw)
    got = to_np32(Y)[np.ix_(rm, rn)]
    r = assert_within(got, ref, bound, "fp8 prefill shape")
    print(f"prefill shape: worst err/bound {r:.3e}")
    # bf16 output: the binary32 result rounded to nearest even
    gb = to_np32(Yb)[np.ix_(rm, rn)]
    assert np.array_equal(gb, to_np32(torch.from_numpy(got).to(torch.bfloat16)))


def test_quantize_rows_near_midpoints_general_scales():
    # arbitrary row maxima (scales that are not powers of two); the other values are E4M3
    # midpoints times the row's binary64 scale, rounded to binary32 and moved by 0 to 24
    # ulps, so their quotients fall on both sides of every rounding decision the kernel's
    # binary32 path could get wrong
    rng = np.random.default_rng(61)
    pos = oracle.E4M3_VALUES[1:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    rows = []
    for _ in range(256):
        amax = np.float32(rng.uniform(0.5, 4.0) * 2.0 ** rng.integers(-20, 20))
        s = np.float64(amax) / 448.0
        pick = rng.choice(mids, 1023) * rng.choice([-1.0, 1.0], 1023)
        base = (pick * s).astype(np.float32)
        moved = (base.view(np.int32) + rng.integers(-24, 25, 1023).astype(np.int32)).view(np.float32)
        moved = np.clip(moved, -amax, amax).astype(np.float32)
        rows.append(np.concatenate([[amax], moved]).astype(np.float32))
    a = np.stack(rows)
    codes, scales = w4.w4_fp8_quantize_rows(torch.from_numpy(a).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows_fp8_ref(a)
    _check_codes(codes, scales, rc, rs, "near-midpoint rows, general scales")
