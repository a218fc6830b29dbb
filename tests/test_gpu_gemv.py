"""GPU parity of w4_gemv against the oracle (dequantize, then dot, in fp64).

Bar: |y_gpu - y_ref| <= 1e-3 * sum_k |w_hat[n, k] * x[m, k]| for every checked
output; one-hot inputs and all-zero rows must match exactly.
"""

import numpy as np
import pytest
import torch

import dequant_gemv_w4_amd as w4
import oracle
import synth
from _util import assert_within, check_quant_and_oracle_products, oracle_quant_rows, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _quant_prepare(W):
    p, s, z = w4.w4_quantize(W)
    prep = w4.w4_prepare(p, s, z)
    return prep, (p, s, z)


def _ref_from_oracle(W32, x32, rows=None):
    """Oracle quantization of W (rows) and fp64 products with x."""
    rows = np.arange(W32.shape[0]) if rows is None else rows
    p, s, z = oracle_quant_rows(W32, rows)
    return oracle.gemv_ref(p, s, z, x32), oracle.tolerance_ref(p, s, z, x32), (p, s, z)


def _run(prep, n, k, x, out_dtype=torch.float32):
    y = w4.w4_gemv(prep, n, k, x, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return y


def test_single_layer_f32_activations():
    w, x = synth.page_single_layer(4096, 4096)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = _run(prep, 4096, 4096, torch.from_numpy(x).to(DEV))
    yr, bound, _ = _ref_from_oracle(w, x)
    r = assert_within(to_np32(y), yr, bound, "4096x4096 f32 x")
    print(f"worst err/bound {r:.3e}")


@pytest.mark.parametrize("xdtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("m", [1, 3, 16])
def test_one_hot_columns_exact(xdtype, m):
    rng = np.random.default_rng(1)
    n, k = 300, 4096
    W = torch.from_numpy((0.02 * rng.standard_normal((n, k))).astype(np.float32)).to(DEV)
    prep, (p, s, z) = _quant_prepare(W)
    cols = rng.choice(k, m, replace=False)
    x = torch.zeros(m, k, dtype=xdtype, device=DEV)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = to_np32(_run(prep, n, k, x))
    wh = oracle.dequant_ref(p.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy())
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), wh[:, c]), f"column {c}"


@pytest.mark.parametrize("matrix", synth.MATRIX_ORDER)
def test_llama7b_layer_with_outlier_channels(matrix):
    W, x = synth.llama7b_layer_matrix(matrix, device=DEV)
    n, k = W.shape
    prep, _ = _quant_prepare(W)
    y = _run(prep, n, k, x)
    yr, bound, _ = _ref_from_oracle(to_np32(W), to_np32(x))
    r = assert_within(to_np32(y), yr, bound, f"7B {matrix}")
    print(f"{matrix}: worst err/bound {r:.3e}")


@pytest.mark.parametrize("matrix", synth.MATRIX_ORDER)
def test_llama70b_layer_every_output(matrix):
    # the 70B-shaped layer: every code of the matrix bit-exact, and every output at
    # M = 1, 2, 3, 4, 8 and 16 against the oracle
    W, x16 = synth.llama70b_layer_matrix(matrix, device=DEV, m=16)
    n, k = W.shape
    p, s, z = w4.w4_quantize(W)
    prep = w4.w4_prepare(p, s, z)
    x32 = to_np32(x16)
    yr, bound = check_quant_and_oracle_products(W, p, s, z, x32, what=f"70B {matrix}")
    del W
    for m in (1, 2, 3, 4, 8, 16):
        y = to_np32(_run(prep, n, k, x16[:m].contiguous()))
        r = assert_within(y, yr[:m], bound[:m], f"70B {matrix} M={m}")
        print(f"{matrix} M={m}: worst err/bound {r:.3e}")


@pytest.mark.parametrize("n,k", [(4096, 4096), (4094, 4096), (1030, 8192), (2050, 2048)])
def test_one_step_workgroups(n, k):
    """Small matrices at M = 1 run workgroups of four rows: every output against the oracle,
    with a ragged last workgroup (N not a multiple of 4), for binary32 x, and for bf16 x both
    ordinary and wide enough in its first 1024 inputs that those waves take the exact path."""
    rng = np.random.default_rng(n + k)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    x = rng.standard_normal((1, k)).astype(np.float32)
    xw = x.copy()
    xw[:, :1024] = synth.wide_range_activations(1, 1024, seed=n)
    for label, xv, dt in (("normal x", x, torch.bfloat16), ("partly wide x", xw, torch.bfloat16),
                          ("binary32 x", xw, torch.float32)):
        xb = torch.from_numpy(xv).to(dt)
        yr, bound, _ = _ref_from_oracle(w, to_np32(xb))
        y = _run(prep, n, k, xb.to(DEV))
        r = assert_within(to_np32(y), yr, bound, f"{n}x{k} {label}")
        print(f"{n}x{k} {label}: worst err/bound {r:.3e}")


def test_short_last_round_rows():
    # 57344 x 8192 at M = 1, 2 (bf16 x) and M = 1 (binary32 x): the one-row kernel's last
    # round of workgroups takes half the rows of the others.  Dense windows around where the
    # short workgroups begin (row 45056 at 16 + 8 rows per workgroup on 256 CUs) and at the
    # end, plus random rows, against the oracle.
    n, k = 57344, 8192
    W = synth.normal_weights(n, k, 2024, DEV)
    prep, _ = _quant_prepare(W)
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([np.arange(44800, 45312), np.arange(n - 256, n),
                                     rng.choice(n, 64, replace=False)]))
    W32 = to_np32(W[torch.from_numpy(rows).to(DEV)])
    del W
    p, s, z = oracle.quantize_ref(W32)
    x16 = synth.normal_activations(2, k, 2025, DEV)
    x32 = torch.from_numpy(to_np32(x16[:1])).to(DEV) * 0.5 + 0.1234567
    for x in (x16[:1].contiguous(), x16, x32):
        m = x.shape[0]
        y = to_np32(_run(prep, n, k, x))
        xr = to_np32(x)
        r = assert_within(y[:, rows], oracle.gemv_ref(p, s, z, xr), oracle.tolerance_ref(p, s, z, xr),
                          f"57344x8192 M={m} {x.dtype}")
        print(f"M={m} {x.dtype}: worst err/bound {r:.3e}")


@pytest.mark.parametrize("n,k,m", [(1, 128, 1), (5, 256, 16), (1000, 384, 2), (77, 11008, 1),
                                   (64, 32768, 1), (64, 32768, 5), (4099, 2048, 8),
                                   (77, 11008, 4), (130, 16512, 2), (33, 16512, 3),
                                   (2050, 384, 16), (96, 32768, 16), (40, 32768, 11),
                                   (3, 128, 16), (7, 384, 8), (33, 1152, 4),
                                   (50, 128, 4), (33, 256, 3), (200, 128, 8)])
def test_shapes_and_ragged_edges(n, k, m):
    rng = np.random.default_rng(n + k + m)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = _run(prep, n, k, x.to(DEV))
    yr, bound, _ = _ref_from_oracle(w, to_np32(x))
    assert_within(to_np32(y), yr, bound, f"N={n} K={k} M={m}")


def _sweep_cases(count=24, seed=2026):
    """Seeded (N, K, M, wide) cases: half with N >= 12033 and K <= 1536 (the resident-x kernel
    for 3 <= M <= 16), half with N <= 3000 and K up to 16384 (the one-row and streaming
    kernels), M from 1 to 16, and in about a third x wide in one random span of inputs."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(count):
        if i % 2 == 0:
            n = int(rng.integers(12033, 20000))
            k = 128 * int(rng.integers(1, 13))
        else:
            n = int(rng.integers(1, 3001))
            k = 128 * int(rng.integers(1, 129))
            n = max(1, min(n, 24_000_000 // k))
        m = int(rng.integers(1, 17))
        cases.append((n, k, m, bool(rng.random() < 0.35)))
    return cases


@pytest.mark.parametrize("n,k,m,wide", _sweep_cases())
def test_random_shape_sweep(n, k, m, wide):
    """Every output against the oracle on seeded shapes across the kernels' routing: ragged
    rows, groups per wave and row steps, every M, and waves whose x falls back to bf16."""
    rng = np.random.default_rng(n * 7 + k * 3 + m)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    if wide:
        a = 128 * int(rng.integers(0, k // 128))
        b = min(k, a + 128 * int(rng.integers(1, 5)))
        x[:, a:b] = synth.wide_range_activations(m, b - a, seed=n + k)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = _run(prep, n, k, xb.to(DEV))
    yr, bound, _ = _ref_from_oracle(w, to_np32(xb))
    assert_within(to_np32(y), yr, bound, f"sweep N={n} K={k} M={m} wide={wide}")


@pytest.mark.parametrize("m", [1, 7, 16])
def test_f32_activations_several_rows(m):
    rng = np.random.default_rng(m)
    n, k = 513, 20480
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = rng.standard_normal((m, k)).astype(np.float32)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = _run(prep, n, k, torch.from_numpy(x).to(DEV))
    yr, bound, _ = _ref_from_oracle(w, x)
    assert_within(to_np32(y), yr, bound, f"f32 x M={m}")


def test_bf16_output():
    rng = np.random.default_rng(4)
    n, k, m = 256, 4096, 4
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = _run(prep, n, k, x.to(DEV), out_dtype=torch.bfloat16)
    assert y.dtype == torch.bfloat16
    yr, bound, _ = _ref_from_oracle(w, to_np32(x))
    # the bf16 store adds at most half an ulp of bf16: 8 significant bits, so at most
    # 2^-8 of the value (at the bottom of a binade)
    assert_within(to_np32(y), yr, bound, "bf16 y", extra=np.abs(yr) * 2.0 ** -8)


def test_all_zero_rows_give_exact_zero():
    rng = np.random.default_rng(8)
    n, k = 64, 8192
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[::3] = 0.0
    w[1, :1024] = 0.0
    x = torch.from_numpy(rng.standard_normal((2, k)).astype(np.float32)).to(torch.bfloat16)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = to_np32(_run(prep, n, k, x.to(DEV)))
    assert np.all(y[:, ::3] == 0.0)
    yr, bound, _ = _ref_from_oracle(w, to_np32(x))
    assert_within(y, yr, bound, "rows with zero groups")


def test_deterministic_repeat():
    W, x = synth.llama70b_layer_matrix("q", device=DEV, m=4)
    prep, _ = _quant_prepare(W)
    y1 = _run(prep, 8192, 8192, x).clone()
    y2 = _run(prep, 8192, 8192, x)
    assert torch.equal(y1, y2)


# ---- batched rows on the resident-x kernel (K <= 8192 and enough rows per workgroup): ragged
# group counts (K = 1152: a wave with four of its eight groups), ragged N, several M

@pytest.mark.parametrize("n,k,m", [(20000, 1152, 3), (12300, 1152, 4), (12300, 1152, 16),
                                   (12289, 4096, 5), (16001, 128, 3), (16001, 128, 16),
                                   (13000, 256, 8), (12100, 384, 12)])
def test_batched_resident_x_shapes_full(n, k, m):
    rng = np.random.default_rng(n + k + m)
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = _run(prep, n, k, x.to(DEV))
    yr, bound, _ = _ref_from_oracle(w, to_np32(x))
    r = assert_within(to_np32(y), yr, bound, f"resident-x N={n} K={k} M={m}")
    print(f"N={n} K={k} M={m}: worst err/bound {r:.3e}")


def test_batched_resident_x_sampled_rows_k8192():
    n, k, m = 20000, 8192, 16
    W = synth.normal_weights(n, k, 777, DEV)
    x16 = synth.normal_activations(m, k, 778, DEV)
    prep, _ = _quant_prepare(W)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 15, 16, n - 1], rng.choice(n, 256, replace=False)]))
    p, s, z = oracle.quantize_ref(to_np32(W[torch.from_numpy(rows).to(DEV)]))
    x32 = to_np32(x16)
    for mm in (3, 4, 8, 16):
        y = to_np32(_run(prep, n, k, x16[:mm].contiguous()))
        assert_within(y[:, rows], oracle.gemv_ref(p, s, z, x32[:mm]),
                      oracle.tolerance_ref(p, s, z, x32[:mm]), f"resident-x sampled M={mm}")


@pytest.mark.parametrize("k", [8192, 8320])
@pytest.mark.parametrize("m", [4, 16])
def test_batched_routing_boundary_sampled_rows(k, m):
    """K = 64 groups (the most the resident-x kernel holds) and 65 groups (the streaming
    kernel) at the same N: sampled rows, including both ends of the last workgroup."""
    n = 12500
    W = synth.normal_weights(n, k, 900 + k, DEV)
    x16 = synth.normal_activations(m, k, 901 + k, DEV)
    prep, _ = _quant_prepare(W)
    rng = np.random.default_rng(k + m)
    rows = np.unique(np.concatenate([[0, 1, 15, 16, 47, 48, n - 17, n - 16, n - 1],
                                     rng.choice(n, 200, replace=False)]))
    p, s, z = oracle.quantize_ref(to_np32(W[torch.from_numpy(rows).to(DEV)]))
    x32 = to_np32(x16)
    y = to_np32(_run(prep, n, k, x16))
    assert_within(y[:, rows], oracle.gemv_ref(p, s, z, x32), oracle.tolerance_ref(p, s, z, x32),
                  f"N={n} K={k} M={m} sampled")


def test_batched_resident_x_one_hot_exact():
    rng = np.random.default_rng(11)
    n, k, m = 12300, 1152, 16
    W = torch.from_numpy((0.02 * rng.standard_normal((n, k))).astype(np.float32)).to(DEV)
    prep, (p, s, z) = _quant_prepare(W)
    cols = rng.choice(k, m, replace=False)
    x = torch.zeros(m, k, dtype=torch.bfloat16, device=DEV)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = to_np32(_run(prep, n, k, x))
    wh = oracle.dequant_ref(p.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy())
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), wh[:, c]), f"column {c}"


def test_batched_resident_x_zero_rows_exact():
    rng = np.random.default_rng(12)
    n, k, m = 20000, 1152, 3
    w = (0.02 * rng.standard_normal((n, k))).astype(np.float32)
    w[::3] = 0.0
    w[1, :512] = 0.0
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    prep, _ = _quant_prepare(torch.from_numpy(w).to(DEV))
    y = to_np32(_run(prep, n, k, x.to(DEV)))
    assert np.all(y[:, ::3] == 0.0)
    yr, bound, _ = _ref_from_oracle(w, to_np32(x))
    assert_within(y, yr, bound, "resident-x rows with zero groups")


def test_decode_step_graph_replays_match_eager():
    """A captured decode step (every w4_gemv of two 70B-shaped layers, M=1 and M=4) gives,
    on every replay, the bits of the eager launches; eager work and synchronizations run
    between the replays."""
    from dequant_gemv_w4_amd.decode import DecodeStep, GemvCall

    shapes = synth.LLAMA70B_FUSED_SHAPES
    preps = {}
    for layer in range(2):
        for name in synth.FUSED_ORDER:
            n, k = shapes[name]
            W = synth.normal_weights(n, k, synth.seed_for(3, synth.FUSED_PARTS[name][0], layer) + 7, DEV)
            preps[(layer, name)] = _quant_prepare(W)[0]
            del W
    for m in (1, 4):
        xs = {8192: synth.normal_activations(m, 8192, 901, DEV),
              28672: synth.normal_activations(m, 28672, 902, DEV)}
        calls = [GemvCall(preps[(layer, name)], shapes[name][0], shapes[name][1],
                          xs[shapes[name][1]],
                          torch.empty(m, shapes[name][0], dtype=torch.float32, device=DEV))
                 for layer in range(2) for name in synth.FUSED_ORDER]
        step = DecodeStep(calls)
        step.run_eager()
        torch.cuda.synchronize()
        eager = [c.y.clone() for c in calls]
        step.capture()
        for rep in range(3):
            for c in calls:
                c.y.fill_(float("nan"))
            torch.cuda.synchronize()
            step.run()
            torch.cuda.synchronize()
            for i, c in enumerate(calls):
                assert torch.equal(c.y, eager[i]), f"M={m} replay {rep} call {i}"

