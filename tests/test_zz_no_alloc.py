"""w4_gemm_noalloc (fixed device workspace, nothing allocated) against w4_gemm.

Two calls in a row on the same GPU, the second with a smaller input, so the second runs
on the workspace the first left behind.  Each call's Y must equal w4_gemm's Y on the same
operands bit for bit (both run the same kernels), and sampled outputs must lie within the
oracle's bound.  Both calls hold rows of X outside the binary16 window, at different row
indices, so a window flag left over from the first call would show in the second.
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


def _weights(n, k, seed):
    w = synth.normal_weights(n, k, seed, DEV)
    p, s, z = w4.w4_quantize(w)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(seed).choice(n, 94, replace=False)]))
    ref = oracle.quantize_ref(to_np32(w[torch.from_numpy(rows).to(DEV)]))
    return w4.w4_prepare(p, s, z), rows, ref


def _x(m, k, wide_rows, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k)).astype(np.float32)
    wide = synth.wide_range_activations(len(wide_rows), k, seed=seed + 1)
    x[wide_rows] = wide
    return torch.from_numpy(x).to(DEV).to(torch.bfloat16)


def _one_call(prep, n, k, X, rows, ref, out_dtype, what):
    Y = torch.full((X.shape[0], n), float("nan"), dtype=out_dtype, device=DEV)
    w4.w4_gemm_noalloc(prep, n, k, X, Y)
    Y_ref = w4.w4_gemm(prep, n, k, X, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_ref), f"{what}: differs from w4_gemm"
    p, s, z = ref
    x32 = to_np32(X)
    yr = oracle.gemv_ref(p, s, z, x32)
    bound = oracle.tolerance_ref(p, s, z, x32)
    # a bf16 store adds at most half an ulp of bf16: 2^-8 of the value at worst
    extra = (np.abs(yr) + bound) * 2.0 ** -8 if out_dtype == torch.bfloat16 else None
    assert_within(to_np32(Y)[:, rows], yr, bound, what, extra=extra)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_noalloc_gemm_two_calls_second_smaller(out_dtype):
    n, k = 1280, 8192
    prep, rows, ref = _weights(n, k, 501)
    # first call: 256 rows (two row tiles), wide rows 5 and 200
    X1 = _x(256, k, [5, 200], 502)
    assert w4.w4_gemm_workspace_bytes(256, n, k) <= w4.GEMM_NOALLOC_MAX_WORKSPACE
    _one_call(prep, n, k, X1, rows, ref, out_dtype, "first call M=256")
    # second call: 37 rows (ragged tile), row 5 ordinary now, row 7 wide
    X2 = _x(37, k, [7], 503)
    _one_call(prep, n, k, X2, rows, ref, out_dtype, "second call M=37")


def test_noalloc_gemm_largest_workspace_and_refusal():
    # the largest prefill shape that fits the fixed workspace (M = 256 at K = 28672,
    # about 14 MiB), then one row more than fits: refused, Y untouched
    n, k = 512, 28672
    prep, rows, ref = _weights(n, k, 511)
    X = _x(256, k, [3], 512)
    _one_call(prep, n, k, X, rows, ref, torch.float32, "M=256 K=28672")
    m_over = w4.GEMM_NOALLOC_MAX_WORKSPACE // (2 * k) + 1
    assert w4.w4_gemm_workspace_bytes(m_over, n, k) > w4.GEMM_NOALLOC_MAX_WORKSPACE
    Xo = torch.zeros(m_over, k, dtype=torch.bfloat16, device=DEV)
    Yo = torch.full((m_over, n), 3.0, dtype=torch.float32, device=DEV)
    with pytest.raises(w4.W4Error) as err:
        w4.w4_gemm_noalloc(prep, n, k, Xo, Yo)
    assert err.value.status == 7
    torch.cuda.synchronize()
    assert bool((Yo == 3.0).all())
