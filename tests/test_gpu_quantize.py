"""GPU parity of w4_quantize and the layout permutation (bit-exact against the oracle)."""

import numpy as np
import pytest
import torch

import dequant_gemv_w4_amd as w4
import oracle
import synth
from _util import assert_quant_equal, oracle_quant_rows, quant_arrays_np, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu_quant(W):
    status = torch.zeros(1, dtype=torch.int32, device=W.device)
    p, s, z = w4.w4_quantize(W, status=status)
    torch.cuda.synchronize()
    return quant_arrays_np(p, s, z), int(status.item())


def test_single_layer_4096_bit_exact():
    w, _ = synth.page_single_layer(4096, 4096)
    gpu, st = _gpu_quant(torch.from_numpy(w).to(DEV))
    assert st == 0
    assert_quant_equal(gpu, oracle.quantize_ref(w), "4096x4096 page draws")


def _edge_rows():
    rng = np.random.default_rng(5)
    rows = []
    # hand-derived tie groups repeated over a 128-group
    for vals in ([-6.5, 8.5, 2.5, -2.5, 0.5, -0.5, 0.0, 1.5], [-1.5, -0.75, -0.05, 0.0],
                 [3.0] * 4, [-3.0] * 4, [0.0] * 4):
        rows.append(np.array(vals * (128 // len(vals)), dtype=np.float32))
    # random groups whose quotients land on exact halves: multiples of s/2 with s = 1
    t = rng.integers(-15, 16, 128).astype(np.float32) / 2
    t[0], t[1] = -7.5, 7.5
    rows.append(t)
    # subnormal ranges, including scales that underflow to 0 in f32 and in fp16
    sub = np.float32(2.0 ** -149)
    rows.append(np.array([-3 * sub, sub, 0.0, 2 * sub] * 32, dtype=np.float32))
    rows.append(np.array([sub, 2 * sub, 0.0, sub] * 32, dtype=np.float32))
    rows.append((rng.standard_normal(128) * 1e-39).astype(np.float32))
    rows.append((rng.standard_normal(128) * 1e-9).astype(np.float32))
    # one-signed and skewed groups, outliers
    rows.append(np.abs(rng.standard_normal(128)).astype(np.float32))
    rows.append(-np.abs(rng.standard_normal(128)).astype(np.float32))
    o = (0.02 * rng.standard_normal(128)).astype(np.float32)
    o[17] = 3.0
    rows.append(o)
    # two groups per row: pad every row to 256 with a random group
    out = []
    for r in rows:
        out.append(np.concatenate([r, (0.02 * rng.standard_normal(128)).astype(np.float32)]))
    return np.stack(out)


def test_edge_groups_bit_exact():
    w = _edge_rows()
    gpu, st = _gpu_quant(torch.from_numpy(w).to(DEV))
    assert_quant_equal(gpu, oracle.quantize_ref(w), "edge groups")
    assert st & w4.STATUS_SCALE_ZERO          # fp16 scale underflow reported
    assert not st & w4.STATUS_NONFINITE


def test_bf16_weights_bit_exact():
    rng = np.random.default_rng(9)
    w = torch.from_numpy((0.02 * rng.standard_normal((37, 384))).astype(np.float32)).to(torch.bfloat16)
    gpu, st = _gpu_quant(w.to(DEV))
    assert st == 0
    assert_quant_equal(gpu, oracle.quantize_ref(to_np32(w)), "bf16 W, ragged 37x384")


def test_status_bits():
    w = torch.zeros(2, 256, device=DEV)
    w[0, 3] = float("nan")
    _, st = _gpu_quant(w)
    assert st & w4.STATUS_NONFINITE
    w = torch.zeros(1, 128, device=DEV)
    w[0, 0], w[0, 1] = -1e6, 1e6                    # scale 133333 > fp16 max
    _, st = _gpu_quant(w)
    assert st & w4.STATUS_SCALE_OVERFLOW


@pytest.mark.parametrize("matrix", synth.MATRIX_ORDER)
def test_llama7b_matrices_bit_exact(matrix):
    W, _ = synth.llama7b_layer_matrix(matrix, device=DEV)
    gpu, st = _gpu_quant(W)
    assert st == 0
    assert_quant_equal(gpu, oracle.quantize_ref(to_np32(W)), f"7B {matrix}")


@pytest.mark.parametrize("matrix", synth.MATRIX_ORDER)
def test_llama70b_matrices_sampled_rows_bit_exact(matrix):
    W, _ = synth.llama70b_layer_matrix(matrix, device=DEV)
    gpu, st = _gpu_quant(W)
    assert st == 0
    n = W.shape[0]
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 384, replace=False)]))
    Wr = to_np32(W[torch.from_numpy(rows).to(DEV)])
    ref = oracle.quantize_ref(Wr)
    gp, gs, gz = gpu
    assert_quant_equal((gp[rows], gs[rows], gz[rows]), ref, f"70B {matrix} sampled rows")


def test_prepare_unprepare_round_trip_random_bytes():
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    for n, k in [(1, 128), (37, 384), (1024, 8192), (8192, 11008 // 128 * 128)]:
        packed = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device=DEV, generator=g)
        scales = torch.randint(-32768, 32767, (n, k // 128), dtype=torch.int16, device=DEV,
                               generator=g).view(torch.float16)
        zeros = torch.randint(0, 256, (n, k // 128), dtype=torch.uint8, device=DEV, generator=g)
        prep = w4.w4_prepare(packed, scales, zeros)
        assert prep.numel() == w4.w4_prepared_bytes(n, k)
        p2, s2, z2 = w4.w4_unprepare(prep, n, k)
        torch.cuda.synchronize()
        assert torch.equal(p2, packed)
        assert torch.equal(s2.view(torch.int16), scales.view(torch.int16))
        assert torch.equal(z2, zeros)
        # the prepared words are a permutation of the canonical nibbles
        assert not torch.equal(prep[: packed.numel()], packed.flatten()) or n * k < 256


def test_page_error_matrix_bit_exact_and_its_error():
    """The seeded 256 x 1024 matrix of page "Quantization", section "Code" (eight 0.6
    outliers) quantized by the library: bit-exact codes, so the asymmetric g128 error of
    the product path is the oracle's (the page's "Try it" item 1 asks for it)."""
    from oracle import quant_error

    w32 = synth.page_error_matrix().astype(np.float32)
    gpu, st = _gpu_quant(torch.from_numpy(w32).to(DEV))
    assert st == 0
    ref = oracle.quantize_ref(w32)
    assert_quant_equal(gpu, ref, "page error matrix")
    db, rel = quant_error.sqnr_db(w32.astype(np.float64), oracle.dequant_ref(*gpu))
    print(f"asymmetric g128 on the page matrix: SQNR {db:.2f} dB, relative RMS {100 * rel:.2f}%")
    sym_db = [r[2] for r in quant_error.table(synth.page_error_matrix()) if r[0] == "INT4 group 128"][0]
    assert db > sym_db


# ---- symmetric variant (page "Quantization" › "How it really works"): bit-exact codes,
# scales and zeros, and the products of the unchanged GEMV/GEMM kernels on its output

def _gpu_quant_sym(W):
    status = torch.zeros(1, dtype=torch.int32, device=W.device)
    p, s, z = w4.w4_quantize_symmetric(W, status=status)
    torch.cuda.synchronize()
    return quant_arrays_np(p, s, z), int(status.item())


def test_symmetric_bit_exact_edges_and_page_matrix():
    rng = np.random.default_rng(21)
    rows = []
    # exact half ties (largest magnitude 7 makes the step 1), zeros, one sign, subnormals
    t = rng.integers(-14, 15, 128).astype(np.float32) / 2
    t[0] = 7.0
    rows.append(t)
    rows.append(np.zeros(128, dtype=np.float32))
    rows.append(np.abs(rng.standard_normal(128)).astype(np.float32))
    rows.append(-np.abs(rng.standard_normal(128)).astype(np.float32))
    rows.append((rng.standard_normal(128) * 1e-39).astype(np.float32))
    rows.append(np.array([2.0 ** -149, 0.0, -(2.0 ** -148), 0.0] * 32, dtype=np.float32))
    o = (0.02 * rng.standard_normal(128)).astype(np.float32)
    o[9] = -3.0
    rows.append(o)
    w = np.stack([np.concatenate([r, (0.02 * rng.standard_normal(128)).astype(np.float32)])
                  for r in rows])
    gpu, st = _gpu_quant_sym(torch.from_numpy(w).to(DEV))
    assert_quant_equal(gpu, oracle.quantize_symmetric_ref(w), "symmetric edge groups")
    wp = synth.page_error_matrix().astype(np.float32)
    gpu, st = _gpu_quant_sym(torch.from_numpy(wp).to(DEV))
    assert st == 0
    assert_quant_equal(gpu, oracle.quantize_symmetric_ref(wp), "symmetric page matrix")


def test_symmetric_70b_rows_bit_exact_and_bf16_input():
    W = synth.normal_weights(28672, 8192, synth.seed_for(3, "gate"), DEV)
    rng = np.random.default_rng(22)
    rows = np.unique(np.concatenate([[0, 28671], rng.choice(28672, 254, replace=False)]))
    gpu, st = _gpu_quant_sym(W)
    assert st == 0
    ref = oracle.quantize_symmetric_ref(to_np32(W[torch.from_numpy(rows).to(DEV)]))
    assert_quant_equal(tuple(a[rows] for a in gpu), ref, "symmetric 70B gate rows")
    Wb = W[:256].to(torch.bfloat16)
    gpu, st = _gpu_quant_sym(Wb)
    assert_quant_equal(gpu, oracle.quantize_symmetric_ref(to_np32(Wb)), "symmetric bf16 W")


def test_symmetric_weights_through_gemv_and_gemm():
    from _util import assert_within
    rng = np.random.default_rng(23)
    n, k = 1000, 2048
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    p, s, z = w4.w4_quantize_symmetric(torch.from_numpy(w).to(DEV))
    prep = w4.w4_prepare(p, s, z)
    rp, rs, rz = oracle.quantize_symmetric_ref(w)
    for m in (1, 3, 8, 16):
        x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
        x32 = to_np32(x)
        y = to_np32(w4.w4_gemv(prep, n, k, x.to(DEV)))
        assert_within(y, oracle.gemv_ref(rp, rs, rz, x32), oracle.tolerance_ref(rp, rs, rz, x32),
                      f"symmetric GEMV M={m}")
    X = torch.from_numpy(rng.standard_normal((130, k)).astype(np.float32)).to(torch.bfloat16)
    x32 = to_np32(X)
    Y = to_np32(w4.w4_gemm(prep, n, k, X.to(DEV)))
    assert_within(Y, oracle.gemv_ref(rp, rs, rz, x32), oracle.tolerance_ref(rp, rs, rz, x32),
                  "symmetric GEMM")



def _near_half_rows(rng, rows: int, symmetric: bool, max_ulps: int = 4):
    """Groups whose binary32 quotients w / s lie on or within a few ulps of k + 1/2, for
    scales that are not powers of two.  The first one or two entries fix the group's range;
    the others are (k + 1/2) * s rounded to binary32 and moved by up to max_ulps ulps."""
    out = []
    for _ in range(rows):
        if symmetric:
            amax = np.float32(rng.uniform(0.01, 2.0))
            s = np.float32(amax / np.float32(7))
            lo, hi = -amax, amax
            ks = rng.integers(-8, 7, 127)
        else:
            lo = np.float32(-rng.uniform(0.01, 2.0))
            hi = np.float32(rng.uniform(0.01, 2.0))
            s = np.float32(np.float32(hi - lo) / np.float32(15))
            ks = rng.integers(-15, 15, 126)
        base = ((ks + 0.5) * np.float64(s)).astype(np.float32)
        moved = (base.view(np.int32) + rng.integers(-max_ulps, max_ulps + 1, base.size).astype(np.int32)).view(np.float32)
        moved = np.clip(moved, lo, hi).astype(np.float32)
        head = [hi] if symmetric else [lo, hi]
        out.append(np.concatenate([np.array(head, dtype=np.float32), moved]))
    return np.stack(out)


def _half_distance(w, symmetric: bool):
    """|w / s - nearest half| in binary32 for every weight after the range-fixing entries."""
    w = w.astype(np.float32)
    if symmetric:
        s = (np.abs(w).max(axis=1) / np.float32(7)).astype(np.float32)
    else:
        s = ((np.maximum(w.max(axis=1), 0) - np.minimum(w.min(axis=1), 0)) / np.float32(15)).astype(np.float32)
    q = (w / s[:, None]).astype(np.float32)
    return np.abs(q - (np.floor(q) + np.float32(0.5)))


@pytest.mark.parametrize("symmetric,max_ulps", [(False, 4), (True, 4), (False, 24), (True, 24)])
def test_quotients_on_and_near_halves_bit_exact(symmetric, max_ulps):
    rng = np.random.default_rng((31 if symmetric else 30) + max_ulps)
    w = _near_half_rows(rng, 512, symmetric, max_ulps)
    d = _half_distance(w, symmetric)
    # the draw holds exact ties and quotients off them on both sides, inside the kernel's
    # window of 2^-17 around each half (exact division) and, with 24 ulps, just outside it
    assert np.count_nonzero(d == 0) > 100
    assert np.count_nonzero((d > 0) & (d < 2.0 ** -17)) > 1000
    if max_ulps > 8:
        assert np.count_nonzero((d > 2.0 ** -17) & (d < 2.0 ** -15)) > 1000
    gpu, st = (_gpu_quant_sym if symmetric else _gpu_quant)(torch.from_numpy(w).to(DEV))
    assert st == 0
    ref = oracle.quantize_symmetric_ref(w) if symmetric else oracle.quantize_ref(w)
    assert_quant_equal(gpu, ref, "quotients on and near halves" + (" (symmetric)" if symmetric else ""))
