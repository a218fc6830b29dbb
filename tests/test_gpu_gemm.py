"""GPU parity of w4_gemm (binary16 MFMA on exact q - zero codes) against the oracle."""

import numpy as np
import pytest
import torch

import dequant_gemv_w4_amd as w4
import oracle
import synth
from _util import assert_within, check_quant_and_oracle_products, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _prep(W):
    p, s, z = w4.w4_quantize(W)
    return w4.w4_prepare(p, s, z)


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (200, 300, 384), (128, 128, 8192), (257, 129, 1024)])
def test_small_full(m, n, k):
    rng = np.random.default_rng(m * 7 + n)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    X = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    prep = _prep(torch.from_numpy(w).to(DEV))
    Y = w4.w4_gemm(prep, n, k, X.to(DEV))
    torch.cuda.synchronize()
    p, s, z = oracle.quantize_ref(w)
    x32 = to_np32(X)
    r = assert_within(to_np32(Y), oracle.gemv_ref(p, s, z, x32), oracle.tolerance_ref(p, s, z, x32),
                      f"GEMM M={m} N={n} K={k}")
    print(f"worst err/bound {r:.3e}")


def test_prefill_shape_rows_and_full_sub_gemm():
    # the prefill shape (M 4096, K 8192, N 28672): every code bit-exact; 64 seeded rows of Y
    # with all 28672 columns; and a full M = 256 product, every output
    W, X = synth.prefill_operands(device=DEV)
    n, k = W.shape
    m = X.shape[0]
    p, s, z = w4.w4_quantize(W)
    prep = w4.w4_prepare(p, s, z)
    rng = np.random.default_rng(31)
    mrows = np.unique(np.concatenate([[0, m - 1], rng.choice(np.arange(1, m - 1), 62, replace=False)]))
    assert mrows.size == 64
    x32 = to_np32(X[torch.from_numpy(mrows).to(DEV)])
    x256 = to_np32(X[:256])
    yr, bound = check_quant_and_oracle_products(W, p, s, z, np.concatenate([x32, x256]),
                                                what="prefill W")
    del W
    Y = w4.w4_gemm(prep, n, k, X)
    torch.cuda.synchronize()
    r = assert_within(to_np32(Y)[mrows], yr[:64], bound[:64], "prefill 4096x8192x28672, 64 rows")
    print(f"64 rows x all columns: worst err/bound {r:.3e}")
    del Y
    Y256 = w4.w4_gemm(prep, n, k, X[:256].contiguous())
    torch.cuda.synchronize()
    r = assert_within(to_np32(Y256), yr[64:], bound[64:], "prefill M=256 sub-GEMM")
    print(f"M=256 sub-GEMM: worst err/bound {r:.3e}")


def test_large_k_operand_offsets():
    """K = 65536 (512 groups): the stage loads address each tile's X' rows and weight columns
    with 32-bit offsets from a uniform base; ragged M and N put clamped rows and columns in
    the last tiles.  Every output against the oracle."""
    rng = np.random.default_rng(77)
    n, k, m = 300, 65536, 130
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    X = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    prep = _prep(torch.from_numpy(w).to(DEV))
    Y = w4.w4_gemm(prep, n, k, X.to(DEV))
    torch.cuda.synchronize()
    p, s, z = oracle.quantize_ref(w)
    x32 = to_np32(X)
    r = assert_within(to_np32(Y), oracle.gemv_ref(p, s, z, x32), oracle.tolerance_ref(p, s, z, x32),
                      f"GEMM M={m} N={n} K={k}")
    print(f"worst err/bound {r:.3e}")


def test_gemm_deterministic():
    rng = np.random.default_rng(2)
    w = torch.from_numpy((0.02 * rng.standard_normal((512, 2048))).astype(np.float32)).to(DEV)
    X = torch.from_numpy(rng.standard_normal((300, 2048)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    prep = _prep(w)
    y1 = w4.w4_gemm(prep, 512, 2048, X).clone()
    y2 = w4.w4_gemm(prep, 512, 2048, X)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_one_hot_rows_and_zero_weight_rows_exact():
    """The B operand is the exact q - zero of every code and the group term is scale16 * P
    (page "Weight quantization", section "How it works"), so a one-hot row of X returns a
    dequantized weight column exactly, and weight rows that are all zero give exactly 0 for
    any X."""
    rng = np.random.default_rng(41)
    n, k, m = 300, 1024, 130
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[::7] = 0.0
    w[1, :256] = 0.0
    prep = _prep(torch.from_numpy(w).to(DEV))
    p, s, z = oracle.quantize_ref(w)
    wh = oracle.dequant_ref(p, s, z)
    cols = rng.choice(k, m, replace=True)
    X = torch.zeros(m, k, dtype=torch.bfloat16)
    X[torch.arange(m), torch.from_numpy(cols)] = 1.0
    Y = to_np32(w4.w4_gemm(prep, n, k, X.to(DEV)))
    for i, c in enumerate(cols):
        assert np.array_equal(Y[i].astype(np.float64), wh[:, c]), f"row {i} (column {c})"
    Xr = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    Yr = to_np32(w4.w4_gemm(prep, n, k, Xr.to(DEV)))
    assert np.all(Yr[:, ::7] == 0.0)
    x32 = to_np32(Xr)
    assert_within(Yr, oracle.gemv_ref(p, s, z, x32), oracle.tolerance_ref(p, s, z, x32), "random X")


def test_bf16_output():
    rng = np.random.default_rng(43)
    n, k, m = 384, 2048, 200
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    X = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    prep = _prep(torch.from_numpy(w).to(DEV))
    Y = w4.w4_gemm(prep, n, k, X.to(DEV), out_dtype=torch.bfloat16)
    assert Y.dtype == torch.bfloat16
    p, s, z = oracle.quantize_ref(w)
    x32 = to_np32(X)
    yr = oracle.gemv_ref(p, s, z, x32)
    # the bf16 store adds at most half an ulp of bf16: 8 significant bits, so at most
    # 2^-8 of the value (at the bottom of a binade)
    assert_within(to_np32(Y), yr, oracle.tolerance_ref(p, s, z, x32), "bf16 Y",
                  extra=np.abs(yr) * 2.0 ** -8)

