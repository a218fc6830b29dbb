"""GPU parity of the products on inputs where exact operands matter.

* Sparse groups: 1-3 non-zero weights per group of 128, the rest exact 0.0, one weight
  negative and one positive, so the zero point is neither 0 nor 15 and every zero weight
  encodes to it (page "Weight quantization" › "Code": the range is widened so that 0 stays
  exactly representable).  Activations are about 3 where the codes equal the zero point and
  about 1e-2 at the non-zero weights, so sum |w_hat x| is tiny next to sum |x|: a product
  that carried a bias through the code (128 + q, corrected by zero * sum x) would miss the
  tolerance by orders of magnitude.
* Wide activations: 32-input slices spanning about 2^40, outside the binary16 window of
  the one-row kernel (its exact path then runs) and of the GEMM pre-pass (its fix-up pass
  recomputes the row).

Bar as everywhere: |y - y_ref| <= 1e-3 * sum_k |w_hat[n, k] x[m, k]| for every output,
y_ref the oracle's fp64 dequantize-then-dot; codes bit-exact.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_w4_amd as w4
import oracle
import synth
from _util import assert_quant_equal, assert_within, quant_arrays_np, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (N, K) reaching each product kernel: the one-row kernel at M = 1..3 on every shape; for
# bf16 x at larger M the streaming matrix-core kernel (few rows, or K > 64 groups) and the
# resident-x kernel (K <= 64 groups, at least 48 rows per workgroup over 256 compute units), which
# converts x to binary16 per row and wave and keeps bf16 x where a wave's x does not convert
# exactly
SHAPES = {"small": (300, 1024), "resident": (12288, 1024), "resident_f16": (24576, 4096),
          "stream": (520, 9216)}
M_VALUES = (1, 2, 3, 4, 8, 16)


def _quant_prepare(w):
    p, s, z = w4.w4_quantize(torch.from_numpy(w).to(DEV))
    ref = oracle.quantize_ref(w)
    assert_quant_equal(quant_arrays_np(p, s, z), ref, "codes")
    return w4.w4_prepare(p, s, z), ref


def _check_gemv(prep, ref, n, k, x, what):
    rp, rs, rz = ref
    y = to_np32(w4.w4_gemv(prep, n, k, x))
    xn = to_np32(x)
    return assert_within(y, oracle.gemv_ref(rp, rs, rz, xn), oracle.tolerance_ref(rp, rs, rz, xn), what)


def _check_gemm(prep, ref, n, k, X, what):
    rp, rs, rz = ref
    Y = to_np32(w4.w4_gemm(prep, n, k, X))
    Xn = to_np32(X)
    return assert_within(Y, oracle.gemv_ref(rp, rs, rz, Xn), oracle.tolerance_ref(rp, rs, rz, Xn), what)


@pytest.mark.parametrize("shape", list(SHAPES))
def test_sparse_groups_with_nonzero_zero_point(shape):
    n, k = SHAPES[shape]
    w, pos = synth.sparse_group_weights(n, k, seed=31 + n)
    prep, ref = _quant_prepare(w)
    rp, rs, rz = ref
    # the case at stake: most codes equal a zero point that is neither 0 nor 15
    codes = oracle.unpack_codes(rp)
    zeros_per_input = np.repeat(rz, 128, axis=1)
    assert np.mean(codes == zeros_per_input) > 0.95
    assert np.mean((rz > 0) & (rz < 15)) > 0.5
    x = synth.sparse_group_activations(16, pos, seed=32 + n)
    worst = 0.0
    for dtype in (torch.bfloat16, torch.float32):
        for m in M_VALUES:
            xm = torch.from_numpy(x[:m]).to(DEV).to(dtype).contiguous()
            worst = max(worst, _check_gemv(prep, ref, n, k, xm, f"{shape} M={m} {dtype}"))
    X = torch.from_numpy(np.tile(x, (13, 1))[:200]).to(DEV).to(torch.bfloat16)
    worst = max(worst, _check_gemm(prep, ref, n, k, X, f"{shape} GEMM M=200"))
    print(f"{shape}: worst err/bound {worst:.3e}")


@pytest.mark.parametrize("shape", list(SHAPES))
def test_wide_range_activations(shape):
    n, k = SHAPES[shape]
    rng = np.random.default_rng(41 + n)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    prep, ref = _quant_prepare(w)
    x = synth.wide_range_activations(16, k, seed=42 + n)
    worst = 0.0
    for dtype in (torch.bfloat16, torch.float32):
        for m in M_VALUES:
            xm = torch.from_numpy(x[:m]).to(DEV).to(dtype).contiguous()
            worst = max(worst, _check_gemv(prep, ref, n, k, xm, f"{shape} M={m} {dtype}"))
    # GEMM: odd rows wide (fix-up pass), even rows ordinary (matrix cores)
    X = rng.standard_normal((150, k)).astype(np.float32)
    X[1::2] = np.tile(x, (5, 1))[: X[1::2].shape[0]]
    worst = max(worst, _check_gemm(prep, ref, n, k, torch.from_numpy(X).to(DEV).to(torch.bfloat16),
                                   f"{shape} GEMM M=150"))
    print(f"{shape}: worst err/bound {worst:.3e}")


def test_resident_x_binary16_some_waves_fall_back():
    """The resident-x kernel on 24576 x 4096 (four waves of eight groups, six row steps): x wide
    only in the first 1024 inputs, so the first wave of every workgroup keeps bf16 x and the
    other three convert it to binary16; every output against the oracle at M = 4, 8, 16."""
    n, k = SHAPES["resident_f16"]
    rng = np.random.default_rng(61)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    prep, ref = _quant_prepare(w)
    x = rng.standard_normal((16, k)).astype(np.float32)
    x[:, :1024] = synth.wide_range_activations(16, 1024, seed=62)
    worst = 0.0
    for m in (4, 8, 16):
        xm = torch.from_numpy(x[:m]).to(DEV).to(torch.bfloat16).contiguous()
        worst = max(worst, _check_gemv(prep, ref, n, k, xm, f"resident-x mixed M={m}"))
        # only rows 0..m-1 matter: a wide row among ordinary ones
        xm2 = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
        xm2[m // 2] = torch.from_numpy(x[0]).to(torch.bfloat16)
        worst = max(worst, _check_gemv(prep, ref, n, k, xm2.to(DEV).contiguous(), f"resident-x one wide row M={m}"))
    print(f"resident-x mixed: worst err/bound {worst:.3e}")


@pytest.mark.parametrize("m", [3, 5, 8])
def test_resident_x_few_rows_ragged_groups_and_a_wide_wave(m):
    """The resident-x kernel with up to eight rows of x (x converted where it was staged) on
    12300 x 1152: two waves of five and four groups (slots past a wave's groups read the next
    bytes), a last workgroup of 12 rows (its one row step starts 4 rows back, in the previous
    workgroup's rows, and stores only its own), and x wide in the second wave's inputs only,
    so one wave keeps bf16 x; every output against the oracle."""
    n, k = 12300, 1152
    rng = np.random.default_rng(90 + m)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    prep, ref = _quant_prepare(w)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, 640:] = synth.wide_range_activations(m, k - 640, seed=91 + m)
    xb = torch.from_numpy(x).to(DEV).to(torch.bfloat16).contiguous()
    r = _check_gemv(prep, ref, n, k, xb, f"resident-x few rows M={m}")
    xn = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(DEV).to(torch.bfloat16)
    r = max(r, _check_gemv(prep, ref, n, k, xn.contiguous(), f"resident-x few rows plain M={m}"))
    print(f"M={m}: worst err/bound {r:.3e}")


@pytest.mark.parametrize("m", [3, 4])
def test_streaming_binary16_x_one_wave_falls_back(m):
    """The streaming kernel with up to four rows of x (binary16 x, converted where it was
    staged) on 520 x 9216: eight waves of nine groups (an odd count: the last pair's second
    group lies past the wave's range), x wide only in the first wave's 1152 inputs, so that
    wave keeps bf16 x; every output against the oracle."""
    n, k = SHAPES["stream"]
    rng = np.random.default_rng(80 + m)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    prep, ref = _quant_prepare(w)
    x = rng.standard_normal((m, k)).astype(np.float32)
    x[:, :1152] = synth.wide_range_activations(m, 1152, seed=81 + m)
    xb = torch.from_numpy(x).to(DEV).to(torch.bfloat16).contiguous()
    r = _check_gemv(prep, ref, n, k, xb, f"streaming one wide wave M={m}")
    print(f"M={m}: worst err/bound {r:.3e}")


@pytest.mark.parametrize("n,k,m,wave", [(40000, 8192, 1, 1), (8192, 28672, 1, 5),
                                         (12000, 8192, 2, 2), (4096, 4096, 1, 1)])
def test_one_row_kernel_one_wave_falls_back(n, k, m, wave):
    """The dot2 kernel (M = 1, 2) with x wide only in the inputs of one wave (2048 per wave),
    so that wave of every workgroup takes the exact path while the others stay on binary16 x:
    workgroups of 16 and 8 rows (40000 x 8192: three and one barriers between steps), 32 rows
    of fourteen waves (8192 x 28672: seven), 8 rows at M = 2, and one-step workgroups (4096 x
    4096).  The exact path passes as many barriers as the pipelined one, so the workgroup's
    partial sums are all written before they are combined.  Sampled rows (both ends of every
    kind of workgroup) against the oracle."""
    W = synth.normal_weights(n, k, 500 + n, DEV)
    p, s, z = w4.w4_quantize(W)
    prep = w4.w4_prepare(p, s, z)
    rng = np.random.default_rng(n + m)
    x = rng.standard_normal((m, k)).astype(np.float32)
    a = 2048 * wave
    x[:, a:a + 2048] = synth.wide_range_activations(m, 2048, seed=501 + n)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(n - 40, n),
                                     rng.choice(n, 240, replace=False)]))
    rp, rs, rz = oracle.quantize_ref(to_np32(W[torch.from_numpy(rows).to(DEV)]))
    y = to_np32(w4.w4_gemv(prep, n, k, xb.to(DEV).contiguous()))
    xn = to_np32(xb)
    r = assert_within(y[:, rows], oracle.gemv_ref(rp, rs, rz, xn), oracle.tolerance_ref(rp, rs, rz, xn),
                      f"dot2 one wide wave {n}x{k} M={m}")
    print(f"{n}x{k} M={m}: worst err/bound {r:.3e}")


@pytest.mark.parametrize("m", [4, 5, 7, 13, 16])
def test_resident_x_binary16_ragged_rows(m):
    """The resident-x kernel's binary16 path with a ragged last workgroup (24616 rows: 220
    workgroups of 112 rows, the last with 88, whose loads for the 24 missing rows repeat row
    N-1) and M not a multiple of four; every output against the oracle."""
    n, k = 24616, 4096
    rng = np.random.default_rng(70 + m)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    prep, ref = _quant_prepare(w)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    r = _check_gemv(prep, ref, n, k, x.to(DEV).contiguous(), f"resident-x ragged M={m}")
    print(f"M={m}: worst err/bound {r:.3e}")


def test_zero_weights_and_exact_zero_rows():
    """Rows of exact zeros (zero point 0) and groups of one repeated negative value give
    exact results whatever x is."""
    n, k = 96, 2048
    rng = np.random.default_rng(5)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[3] = 0.0
    w[10, :128] = -0.5     # one-signed group: zero 15, codes 0
    prep, ref = _quant_prepare(w)
    x = (100.0 * rng.standard_normal((16, k))).astype(np.float32)
    for m in (1, 3, 16):
        xm = torch.from_numpy(x[:m]).to(DEV).to(torch.bfloat16)
        y = to_np32(w4.w4_gemv(prep, n, k, xm))
        assert np.all(y[:, 3] == 0.0)
        _check_gemv(prep, ref, n, k, xm, f"M={m}")
    Y = to_np32(w4.w4_gemm(prep, n, k, torch.from_numpy(x).to(DEV).to(torch.bfloat16)))
    assert np.all(Y[:, 3] == 0.0)
