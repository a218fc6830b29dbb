"""Parity of the decode step exactly as the benchmark builds and times it.

The benchmark draws each layer's weights on the GPU, quantizes and prepares them with
q|k|v and gate|up concatenated along N, captures the step into a graph and replays it.
Here two such layers are built with the benchmark's own functions, the step is replayed
at M = 1, 4 and 16, and sampled rows of every output are checked against the oracle on
the same weight rows (drawn again from the same seeds) and the same activations.
"""

import numpy as np
import pytest
import torch

import bench
import oracle
import synth
import dequant_gemv_w4_amd as w4
from _util import assert_quant_equal, assert_within, quant_arrays_np, to_np32

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def test_bench_step_sampled_rows_against_oracle():
    layers = 2
    prepared = bench.build_stack(layers, DEV, fused=True)
    rng = np.random.default_rng(77)
    order = synth.FUSED_ORDER
    shapes = synth.LLAMA70B_FUSED_SHAPES
    # the sampled weight rows, drawn again exactly as build_stack drew them
    refs = {}
    for layer in range(layers):
        for name in order:
            n, k = shapes[name]
            seed = synth.seed_for(4, synth.FUSED_PARTS[name][0], layer) + 10000
            W = synth.normal_weights(n, k, seed, DEV)
            rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 62, replace=False)]))
            refs[(layer, name)] = (rows, oracle.quantize_ref(to_np32(W[torch.from_numpy(rows).to(DEV)])))
            del W
    for m in (1, 4, 16):
        step = bench.make_step(prepared, layers, m, DEV, fused=True)
        step.capture()
        for _ in range(2):
            step.run()
        torch.cuda.synchronize()
        worst = 0.0
        for i, call in enumerate(step.calls):
            layer, name = divmod(i, len(order))
            rows, (p, s, z) = refs[(layer, order[name])]
            x32 = to_np32(call.x)
            r = assert_within(to_np32(call.y)[:, rows], oracle.gemv_ref(p, s, z, x32),
                              oracle.tolerance_ref(p, s, z, x32),
                              f"bench step M={m} layer {layer} {order[name]}")
            worst = max(worst, r)
        print(f"M={m}: worst err/bound {worst:.3e}")
        del step


def test_full_80_layer_step_sampled_rows_against_oracle():
    # the headline workload at its full size: 80 fused layers (about 36 GB resident), M = 1,
    # replayed from the captured graph exactly as the benchmark times it; 512 seeded rows of
    # every matrix of every layer against the oracle (codes and products), and two replays
    # bit-identical
    layers = 80
    prepared = bench.build_stack(layers, DEV, fused=True)
    step = bench.make_step(prepared, layers, 1, DEV, fused=True)
    step.capture()
    step.run()
    torch.cuda.synchronize()
    first = [c.y.clone() for c in step.calls]
    step.run()
    torch.cuda.synchronize()
    assert all(torch.equal(c.y, f) for c, f in zip(step.calls, first)), "replays differ"
    del first
    order = synth.FUSED_ORDER
    shapes = synth.LLAMA70B_FUSED_SHAPES
    rng = np.random.default_rng(80)
    worst = 0.0
    for i, call in enumerate(step.calls):
        layer, j = divmod(i, len(order))
        name = order[j]
        n, k = shapes[name]
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(np.arange(1, n - 1), 510, replace=False)]))
        assert rows.size == 512
        seed = synth.seed_for(4, synth.FUSED_PARTS[name][0], layer) + 10000
        W = synth.normal_weights(n, k, seed, DEV)
        w32 = to_np32(W[torch.from_numpy(rows).to(DEV)])
        del W
        p, s, z = oracle.quantize_ref(w32)
        # the codes the step reads: the prepared matrix taken back to the canonical arrays
        gp, gs, gz = w4.w4_unprepare(prepared[(layer, name)], n, k)
        sel = torch.from_numpy(rows).to(DEV)
        assert_quant_equal(quant_arrays_np(gp[sel], gs[sel], gz[sel]), (p, s, z),
                           f"80-layer step layer {layer} {name} codes")
        del gp, gs, gz
        x32 = to_np32(call.x)
        r = assert_within(to_np32(call.y)[:, rows], oracle.gemv_ref(p, s, z, x32),
                          oracle.tolerance_ref(p, s, z, x32), f"80-layer step layer {layer} {name}")
        worst = max(worst, r)
    print(f"80 layers: worst err/bound {worst:.3e}")


def test_stream_read_probe_reads_without_writing():
    # the bandwidth probe leaves its sink alone unless the folded words equal its fixed
    # word; a zero buffer folds to 0, and a ragged size (not a multiple of the share)
    # must read in bounds
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    for nbytes in (16, 4096 * 16 + 48, 3 << 20):
        buf = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
        w4.w4_stream_read(buf, sink)
        torch.cuda.synchronize()
        assert int(sink.item()) == 7
