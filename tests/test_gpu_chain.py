"""GPU checks of w4_chain_run (persistent multi-stage GEMV launch).

Oracle parity on independent stages with synthetic x; stage ordering checked by a
stage that reads the previous stage's output, compared with a separate w4_gemv
launch on the same device buffer (the oracle never takes GPU outputs as input).
"""

import numpy as np
import pytest
import torch

import dequant_gemv_w4_amd as w4
import oracle
import synth
from _util import assert_within, to_np32
from dequant_gemv_w4_amd.decode import GemvCall, GemvChain

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _prep(W):
    p, s, z = w4.w4_quantize(W)
    return w4.w4_prepare(p, s, z)


def _mat(n, k, seed):
    return synth.normal_weights(n, k, seed, DEV)


def test_independent_stages_match_oracle():
    shapes = [(1000, 8192), (8192, 28672), (77, 4096), (4100, 11008 // 128 * 128), (64, 32768)]
    calls, refs = [], []
    for i, (n, k) in enumerate(shapes):
        W = _mat(n, k, 500 + i)
        x = synth.normal_activations(1, k, 600 + i, DEV)
        y = torch.full((1, n), float("nan"), dtype=torch.float32, device=DEV)
        calls.append(GemvCall(_prep(W), n, k, x, y))
        rng = np.random.default_rng(i)
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, min(n, 200), replace=False)]))
        refs.append((rows, to_np32(W[torch.from_numpy(rows).to(DEV)]), to_np32(x)))
    # two calls per stage, some stages with one
    stages = [[calls[0], calls[2]], [calls[1]], [calls[3], calls[4]]]
    ch = GemvChain(stages)
    ch.run()
    torch.cuda.synchronize()
    assert ch.status() == 0
    for c, (rows, W32, x32) in zip(calls, refs):
        p, s, z = oracle.quantize_ref(W32)
        y = to_np32(c.y)[:, rows]
        r = assert_within(y, oracle.gemv_ref(p, s, z, x32), oracle.tolerance_ref(p, s, z, x32),
                          f"chain N={c.n} K={c.k}")
        print(f"N={c.n} K={c.k}: worst err/bound {r:.3e}")


def test_stage_reads_previous_output():
    # stage 0: y0 = W0 x0 (bf16 out);  stage 1: y1 = W1 y0;  stage 2: y2 = W2 y1
    W0, W1, W2 = _mat(4096, 8192, 701), _mat(8192, 4096, 702), _mat(3000, 8192, 703)
    P0, P1, P2 = _prep(W0), _prep(W1), _prep(W2)
    x0 = synth.normal_activations(1, 8192, 704, DEV)
    y0 = torch.full((1, 4096), float("nan"), dtype=torch.bfloat16, device=DEV)
    y1 = torch.full((1, 8192), float("nan"), dtype=torch.bfloat16, device=DEV)
    y2 = torch.full((1, 3000), float("nan"), dtype=torch.float32, device=DEV)
    ch = GemvChain([[GemvCall(P0, 4096, 8192, x0, y0)], [GemvCall(P1, 8192, 4096, y0, y1)],
                    [GemvCall(P2, 3000, 8192, y1, y2)]])
    for rep in range(3):
        for t in (y0, y1, y2):
            t.fill_(float("nan"))
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        r0 = w4.w4_gemv(P0, 4096, 8192, x0, out_dtype=torch.bfloat16)
        r1 = w4.w4_gemv(P1, 8192, 4096, y0, out_dtype=torch.bfloat16)
        r2 = w4.w4_gemv(P2, 3000, 8192, y1)
        torch.cuda.synchronize()
        # K <= 8192: the chain's per-lane arithmetic and summation order equal w4_gemv's
        assert torch.equal(y0, r0) and torch.equal(y1, r1) and torch.equal(y2, r2), rep


def test_graph_replays_and_repeat_determinism():
    shapes = [(10240, 8192), (8192, 8192), (57344, 8192), (8192, 28672)]
    stages = []
    for i, (n, k) in enumerate(shapes):
        x = synth.normal_activations(1, k, 800 + i, DEV)
        y = torch.empty(1, n, dtype=torch.float32, device=DEV)
        stages.append([GemvCall(_prep(_mat(n, k, 810 + i)), n, k, x, y)])
    ch = GemvChain(stages)
    ch.run()
    torch.cuda.synchronize()
    ref = [c.y.clone() for c in ch.calls]
    ch.capture()
    for rep in range(4):
        for c in ch.calls:
            c.y.zero_()
        ch.run()
        torch.cuda.synchronize()
        assert ch.status() == 0
        for c, r in zip(ch.calls, ref):
            assert torch.equal(c.y, r), f"replay {rep} N={c.n}"
    # eager call between replays
    ch.run_eager()
    torch.cuda.synchronize()
    for c, r in zip(ch.calls, ref):
        assert torch.equal(c.y, r)
