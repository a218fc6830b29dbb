"""Helpers shared by the GPU parity tests (comparison only; no method arithmetic)."""

from __future__ import annotations

import numpy as np

import oracle


def to_np32(t) -> np.ndarray:
    """float32 NumPy copy of a torch tensor (bf16 values convert exactly)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def quant_arrays_np(packed, scales, zeros):
    """Canonical GPU arrays as NumPy (packed uint8, scales float16, zeros uint8)."""
    return (packed.cpu().numpy(), scales.cpu().numpy(), zeros.cpu().numpy())


def assert_quant_equal(gpu, ref, what=""):
    gp, gs, gz = gpu
    rp, rs, rz = ref
    assert gp.shape == rp.shape and gs.shape == rs.shape and gz.shape == rz.shape, what
    bad = np.argwhere(gp != rp)
    assert bad.size == 0, f"{what}: packed differs at {bad[:5].tolist()} (of {len(bad)})"
    bad = np.argwhere(gs.view(np.uint16) != rs.view(np.uint16))
    assert bad.size == 0, f"{what}: scales differ at {bad[:5].tolist()}"
    bad = np.argwhere(gz != rz)
    assert bad.size == 0, f"{what}: zeros differ at {bad[:5].tolist()}"


def assert_within(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what="",
                  extra: np.ndarray | None = None):
    """|y_gpu - y_ref| <= bound (+ extra) elementwise; reports the worst ratio."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    lim = bound if extra is None else bound + extra
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    ok = err <= lim
    if not np.all(ok):
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError(
            f"{what}: {np.count_nonzero(~ok)} outputs out of tolerance; worst at {i}: "
            f"gpu {y_gpu[i]!r} ref {y_ref[i]!r} err {err[i]:.3e} bound {lim[i]:.3e}")
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(lim > 0, err / lim, 0.0)
    return float(ratio.max()) if ratio.size else 0.0


def oracle_quant_rows(W32: np.ndarray, rows):
    """Oracle quantization of selected rows (groups never cross rows)."""
    return oracle.quantize_ref(np.ascontiguousarray(W32[rows]))


def check_quant_and_oracle_products(W, p, s, z, x32: np.ndarray, chunk: int = 2048, what=""):
    """Oracle quantization of every row of the GPU weights W (copied in row chunks), checked
    bit-exact against the GPU's canonical arrays (p, s, z), and the oracle's products with
    x32 [M, K] and their bounds for every row.  Returns (y_ref [M, N], bound [M, N])."""
    n = W.shape[0]
    yr = np.empty((x32.shape[0], n), dtype=np.float64)
    bound = np.empty_like(yr)
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        ref = oracle.quantize_ref(to_np32(W[r0:r1]))
        assert_quant_equal(quant_arrays_np(p[r0:r1], s[r0:r1], z[r0:r1]), ref, f"{what} rows {r0}..{r1}")
        yr[:, r0:r1] = oracle.gemv_ref(*ref, x32)
        bound[:, r0:r1] = oracle.tolerance_ref(*ref, x32)
    return yr, bound
