"""GPU parity of the W8A8 INT8 path (w4_int8_quantize_rows, w4_int8_gemm) against the oracle.

Codes and steps must match the oracle bit for bit; products must lie within
1e-3 * sum_k |x_hat[m, k] * w_hat[n, k]| of the oracle's fp64 product.  The integer sums
are exact, so the output must also equal, bit for bit, the binary32 scaling of the exact
integer dot product of the oracle's codes.
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
    bad = np.argwhere(c != ref_codes)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[0]}"
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32)), f"{what}: steps differ"


def _exact_scaled(cx, sx, cw, sw):
    acc = cx.astype(np.int64) @ cw.astype(np.int64).T
    return (acc.astype(np.float32) * sx[:, None]).astype(np.float32) * sw[None, :]


def test_quantize_rows_bit_exact_edge_rows():
    rng = np.random.default_rng(51)
    a = (rng.standard_normal((300, 1024)) * np.exp(rng.uniform(-20, 20, (300, 1)))).astype(np.float32)
    a[0] = 0.0
    a[1] = 0.0
    a[1, 9] = -5.0                                  # one value: -127
    a[2, :64] = np.arange(-31.5, 32.5, 1.0)          # exact ties at step 1
    a[2, 64:] = 0.25
    a[2, 100] = 127.0
    a[3, :] = np.float32(3.0e38)
    A = torch.from_numpy(a).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    codes, steps = w4.w4_int8_quantize_rows(A, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    rc, rs = oracle.quantize_rows_int8_ref(a)
    _check_codes(codes, steps, rc, rs, "f32 rows")
    assert rc[1, 9] == -127 and rc[2, 0] == -32 and rc[2, 1] == -30


@pytest.mark.parametrize("rows,k", [(77, 8192), (5, 128), (130, 384), (3, 8320), (2, 65536)])
def test_quantize_rows_bf16_activations(rows, k):
    X = synth.normal_activations(rows, k, 5200 + rows, DEV)
    X[:, : max(1, k // 100)] *= 20
    codes, steps = w4.w4_int8_quantize_rows(X.contiguous())
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows_int8_ref(to_np32(X))
    _check_codes(codes, steps, rc, rs, f"bf16 {rows}x{k}")


@pytest.mark.parametrize("m,n,k", [(200, 300, 384), (1, 1, 128), (129, 257, 1024), (64, 4096, 8192),
                                   (3, 5, 65536)])
def test_gemm_full_small(m, n, k):
    X = synth.normal_activations(m, k, 5300 + m, DEV)
    W = synth.normal_weights(n, k, 5301 + n, DEV)
    xq, sx = w4.w4_int8_quantize_rows(X)
    wq, sw = w4.w4_int8_quantize_rows(W)
    Y = w4.w4_int8_gemm(xq, sx, wq, sw)
    torch.cuda.synchronize()
    rcx, rsx = oracle.quantize_rows_int8_ref(to_np32(X))
    rcw, rsw = oracle.quantize_rows_int8_ref(to_np32(W))
    _check_codes(xq, sx, rcx, rsx, "x")
    _check_codes(wq, sw, rcw, rsw, "w")
    got = to_np32(Y)
    r = assert_within(got, oracle.gemm_int8_ref(rcx, rsx, rcw, rsw),
                      oracle.tolerance_int8_ref(rcx, rsx, rcw, rsw), f"int8 gemm {m}x{n}x{k}")
    assert np.array_equal(got, _exact_scaled(rcx, rsx, rcw, rsw)), "int32 sums not exact"
    print(f"{m}x{n}x{k}: worst err/bound {r:.3e}")


def test_prefill_shape_sampled_outputs():
    m, n, k = 4096, 28672, 8192
    X = synth.normal_activations(m, k, 5400, DEV)
    W = synth.normal_weights(n, k, 5401, DEV)
    xq, sx = w4.w4_int8_quantize_rows(X)
    wq, sw = w4.w4_int8_quantize_rows(W)
    Y = w4.w4_int8_gemm(xq, sx, wq, sw)
    Yb = w4.w4_int8_gemm(xq, sx, wq, sw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(53)
    rm = np.unique(np.concatenate([[0, m - 1], rng.choice(m, 62, replace=False)]))
    rn = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 446, replace=False)]))
    x32 = to_np32(X[torch.from_numpy(rm).to(DEV)])
    w32 = to_np32(W[torch.from_numpy(rn).to(DEV)])
    del X, W
    rcx, rsx = oracle.quantize_rows_int8_ref(x32)
    rcw, rsw = oracle.quantize_rows_int8_ref(w32)
    _check_codes(xq[torch.from_numpy(rm).to(DEV)], sx[torch.from_numpy(rm).to(DEV)], rcx, rsx, "x rows")
    _check_codes(wq[torch.from_numpy(rn).to(DEV)], sw[torch.from_numpy(rn).to(DEV)], rcw, rsw, "w rows")
    got = to_np32(Y)[np.ix_(rm, rn)]
    r = assert_within(got, oracle.gemm_int8_ref(rcx, rsx, rcw, rsw),
                      oracle.tolerance_int8_ref(rcx, rsx, rcw, rsw), "int8 prefill shape")
    assert np.array_equal(got, _exact_scaled(rcx, rsx, rcw, rsw)), "int32 sums not exact"
    gb = to_np32(Yb)[np.ix_(rm, rn)]
    assert np.array_equal(gb, to_np32(torch.from_numpy(got).to(torch.bfloat16)))
    print(f"prefill shape: worst err/bound {r:.3e}")


def test_quantize_rows_near_halves_general_scales():
    # arbitrary row maxima; the other values are (k + 1/2) times the row's binary64 step,
    # rounded to binary32 and moved by 0 to 24 ulps (both sides of the kernel's binary32
    # rounding decisions)
    rng = np.random.default_rng(62)
    rows = []
    for _ in range(256):
        amax = np.float32(rng.uniform(0.5, 4.0) * 2.0 ** rng.integers(-20, 20))
        s = np.float64(amax) / 127.0
        k = rng.integers(-127, 127, 1023) + 0.5
        base = (k * s).astype(np.float32)
        moved = (base.view(np.int32) + rng.integers(-24, 25, 1023).astype(np.int32)).view(np.float32)
        moved = np.clip(moved, -amax, amax).astype(np.float32)
        rows.append(np.concatenate([[amax], moved]).astype(np.float32))
    a = np.stack(rows)
    codes, steps = w4.w4_int8_quantize_rows(torch.from_numpy(a).to(DEV))
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_rows_int8_ref(a)
    _check_codes(codes, steps, rc, rs, "near-half rows, general steps")
