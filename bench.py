#!/usr/bin/env python3
"""W4A16 g128 decode benchmark on one MI355X.

Workload (one "step"): a 70B-shaped decode step at batch 1 -- 80 layers, each
with the seven GQA matrices q/o 8192x8192, k/v 1024x8192, gate/up 28672x8192
and down 8192x28672, quantized to asymmetric int4 with group 128 and resident
in HBM in the kernel layout (about 36 GB); every matrix is multiplied once by
its bf16 activation row with w4_gemv, back to back, replayed from one captured
graph.  The headline step stores the same-input matrices concatenated along N
(q|k|v as 10240x8192, gate|up as 57344x8192), so a layer is four launches
(qkv, o, gate_up, down); the step with seven separate launches per layer is
reported beside it.  Weights are N(0, 0.02) and activations N(0, 1), drawn on
the GPU from fixed seeds (synthetic, no checkpoint).

The printed JSON line reports the achieved HBM bandwidth of the step computed
from algorithmic bytes (codes + fp16 scales + byte zeros + activations +
outputs), the roofline fraction against the 8 TB/s HBM peak, and the CPU
oracle's rate on a bounded sample of the same work.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
# HBM bytes per launch of the batch-1 fused step from rocprofv3 counters on the current
# w4_gemv kernel (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by what the counter
# reads for a 256 MiB device copy), or None while the kernel has changed since they were
# taken.
GEMV_STEP_TRAFFIC_BYTES_PER_LAUNCH = 114101898
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
W8_DENSE_TOPS = 5000.0         # MI355X dense fp8 MFMA TFLOP/s, and int8 TOP/s
METRIC = "W4A16 g128 GEMV achieved HBM GB/s (% of peak), 70B layer shapes, batch 1"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=80)
    ap.add_argument("--no-graph", action="store_true", help="launch the 560 GEMVs eagerly")
    ap.add_argument("--skip-extras", action="store_true",
                    help="only the headline step (no batch sweep, per-shape, GEMM, quantizer)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the W4A16 prefill GEMM leg, three timed calls (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 256 MiB device-to-device copy (a known-size kernel that "
                         "scales the byte counters of a profiler run)")
    return ap.parse_args()


def build_stack(layers: int, dev: str, fused: bool = False):
    """Quantize and prepare every matrix of the stack on the GPU (weights drawn there).

    With fused=True the same-input matrices are drawn as one concatenated matrix
    (q|k|v: 10240 x 8192, gate|up: 57344 x 8192), so each group is one launch.
    """
    import torch

    import dequant_gemv_w4_amd as w4
    import synth

    prepared = {}
    t0 = time.time()
    order = synth.FUSED_ORDER if fused else synth.MATRIX_ORDER
    shapes = synth.LLAMA70B_FUSED_SHAPES if fused else synth.LLAMA70B_SHAPES
    for layer in range(layers):
        for name in order:
            n, k = shapes[name]
            seed = synth.seed_for(4, synth.FUSED_PARTS[name][0] if fused else name, layer)
            W = synth.normal_weights(n, k, seed + (10000 if fused else 0), dev)
            p, s, z = w4.w4_quantize(W)
            prepared[(layer, name)] = w4.w4_prepare(p, s, z)
            del W, p, s, z
        if layer % 10 == 9 or layer == layers - 1:
            torch.cuda.synchronize()
            log(f"quantized and prepared {layer + 1}/{layers} layers ({time.time() - t0:.1f} s)")
    return prepared


def make_step(prepared, layers: int, m: int, dev: str, fused: bool = False):
    import torch

    import synth
    from dequant_gemv_w4_amd.decode import DecodeStep, GemvCall

    # activation rows feeding each matrix (the step's inputs; fixed across layers)
    xs = {
        "attn": synth.normal_activations(m, 8192, 40001, dev),
        "o": synth.normal_activations(m, 8192, 40002, dev),
        "mlp": synth.normal_activations(m, 8192, 40003, dev),
        "down": synth.normal_activations(m, 28672, 40004, dev),
    }
    feed = {"q": "attn", "k": "attn", "v": "attn", "o": "o", "gate": "mlp", "up": "mlp",
            "down": "down", "qkv": "attn", "gate_up": "mlp"}
    order = synth.FUSED_ORDER if fused else synth.MATRIX_ORDER
    shapes = synth.LLAMA70B_FUSED_SHAPES if fused else synth.LLAMA70B_SHAPES
    calls = []
    for layer in range(layers):
        for name in order:
            n, k = shapes[name]
            y = torch.empty(m, n, dtype=torch.float32, device=dev)
            calls.append(GemvCall(prepared[(layer, name)], n, k, xs[feed[name]], y))
    return DecodeStep(calls)


def time_step(step, steps: int, warmup: int, per_step: list | None = None) -> float:
    """Milliseconds per step from HIP events on the launch stream.

    The K timed steps run back to back between one start and one end event; when
    per_step is a list, an event is also recorded after every step and the K
    individual step times are appended to it (for median and percentiles).
    """
    import torch
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps)] if per_step is not None else []
    start.record()
    for i in range(steps):
        step.run()
        if marks:
            marks[i].record()
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    if marks:
        prev = start
        for ev in marks:
            per_step.append(prev.elapsed_time(ev))
            prev = ev
    return start.elapsed_time(end) / steps


def percentile(values: list, q: float) -> float:
    v = sorted(values)
    if not v:
        return float("nan")
    pos = (len(v) - 1) * q
    lo = int(pos)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (pos - lo)


def per_shape(prepared, layers: int, dev: str, reps: int = 3, fused: bool = False, m: int = 1,
              with_read: bool = False):
    """Isolated GB/s per matrix shape at batch m: the same shape across all layers, back to back.

    With ``with_read``, also the time of a plain read (w4_stream_read) of the same prepared
    buffers in the same launch pattern, and the ratio of the two.
    """
    import synth
    import dequant_gemv_w4_amd as w4
    from dequant_gemv_w4_amd.decode import DecodeStep, GemvCall
    import torch

    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    order = synth.FUSED_ORDER if fused else synth.MATRIX_ORDER
    shapes = synth.LLAMA70B_FUSED_SHAPES if fused else synth.LLAMA70B_SHAPES
    for name in order:
        n, k = shapes[name]
        x = synth.normal_activations(m, k, 40100, dev)
        calls = [GemvCall(prepared[(layer, name)], n, k, x,
                          torch.empty(m, n, dtype=torch.float32, device=dev))
                 for layer in range(layers)]
        st = DecodeStep(calls)
        st.capture()
        ms = time_step(st, reps, 1)
        out[name] = {"N": n, "K": k, "us_per_call": round(ms * 1000 / layers, 2),
                     "GB/s": round(st.algorithmic_bytes() / (ms * 1e-3) / 1e9, 1)}
        if with_read:
            bufs = [prepared[(layer, name)] for layer in range(layers)]
            for b in bufs:
                w4.w4_stream_read(b, sink)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for b in bufs:
                    w4.w4_stream_read(b, sink)
            g.replay()
            torch.cuda.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            start.record()
            for _ in range(reps):
                g.replay()
            end.record()
            end.synchronize()
            read_us = start.elapsed_time(end) * 1000 / (reps * layers)
            out[name]["read_probe_us_per_call"] = round(read_us, 2)
            out[name]["gemv_vs_read"] = round(read_us / (ms * 1000 / layers), 4)
    return out


def read_ceiling(prepared, layers: int, dev: str, step_ms: float, reps: int = 10):
    """What a kernel that only reads achieves (w4_stream_read, a plain streaming read).

    ``stream``: one 4 GiB buffer read start to end.  ``step_pattern``: every prepared matrix
    of the step read once, in the step's order, as one launch each from one graph: the
    same bytes (layout padding included) in the same launch pattern as the GEMV step, so
    ``gemv_step_vs_pattern`` (pattern time / GEMV step time) says how close the products
    come to a pure read.
    """
    import torch

    import dequant_gemv_w4_amd as w4
    import synth

    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    big = torch.zeros(4 << 30, dtype=torch.uint8, device=dev)
    for _ in range(2):
        w4.w4_stream_read(big, sink)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        w4.w4_stream_read(big, sink)
    end.record()
    end.synchronize()
    stream_gbs = big.numel() * reps / (start.elapsed_time(end) * 1e-3) / 1e9
    del big
    torch.cuda.empty_cache()

    bufs = [prepared[(layer, name)] for layer in range(layers) for name in synth.FUSED_ORDER]
    for b in bufs:
        w4.w4_stream_read(b, sink)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for b in bufs:
            w4.w4_stream_read(b, sink)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    end.synchronize()
    ms = start.elapsed_time(end) / reps
    nbytes = sum(b.numel() for b in bufs)
    return {"stream_GB/s": round(stream_gbs, 1),
            "stream_pct_of_hbm_peak": round(100 * stream_gbs / HBM_PEAK_GBS, 2),
            "step_pattern_ms": round(ms, 4), "step_pattern_bytes": int(nbytes),
            "step_pattern_GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "gemv_step_vs_pattern": round(ms / step_ms, 4)}


def page_layer(dev: str, reps: int = 5, copies: int = 64):
    """The page's single layer: W 4096x4096 and binary32 x from its xorshift draws, M=1.

    ``copies`` prepared copies (64 x 8.8 MB, past the 256 MB MALL) are multiplied back to
    back in one graph, so every call streams its weights from HBM.
    """
    import torch

    import dequant_gemv_w4_amd as w4
    import synth
    from dequant_gemv_w4_amd.decode import DecodeStep, GemvCall

    w, x = synth.page_single_layer(4096, 4096)
    p, s, z = w4.w4_quantize(torch.from_numpy(w).to(dev))
    prep = w4.w4_prepare(p, s, z)
    xt = torch.from_numpy(x).to(dev)
    calls = [GemvCall(prep.clone(), 4096, 4096, xt, torch.empty(1, 4096, dtype=torch.float32, device=dev))
             for _ in range(copies)]
    st = DecodeStep(calls)
    st.capture()
    ms = time_step(st, reps, 1)
    gbs = st.algorithmic_bytes() / (ms * 1e-3) / 1e9
    return {"N": 4096, "K": 4096, "x": "binary32", "copies": copies,
            "us_per_call": round(ms * 1000 / copies, 2), "GB/s": round(gbs, 1),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}


FORMAT_VARIANTS = [  # (group, bf16 scale, zero bits): the storage variants timed at M = 1
    (128, False, 8), (128, True, 8), (128, False, 4), (64, False, 8), (32, False, 8), (32, True, 4),
]


def format_variants(dev: str, reps: int = 5, copies: int = 2, calls: int = 16):
    """w4_gemv_fmt at M = 1 on the 70B gate|up shape (57344 x 8192, bf16 x) per storage format.

    ``copies`` prepared copies (2 x ~240 MB, past the 256 MB MALL) alternate over ``calls``
    products in one graph.  GB/s counts the format's own bytes (codes, 2-byte scales, 4- or
    8-bit zeros per group, x, y); the prepared layout carries every group's scale and zero
    in one 4-byte word.
    """
    import torch

    import dequant_gemv_w4_amd as w4
    import synth
    from dequant_gemv_w4_amd.decode import DecodeStep, GemvCall

    n, k = synth.LLAMA70B_FUSED_SHAPES["gate_up"]
    x = synth.normal_activations(1, k, 40200, dev)
    out = {}
    for group, sbf, zb in FORMAT_VARIANTS:
        f = w4.W4Format.make(group, sbf, zb, False)
        preps = []
        for c in range(copies):
            W = synth.normal_weights(n, k, 40300 + c, dev)
            p, s, z = w4.w4_quantize_fmt(W, f)
            del W
            preps.append(w4.w4_prepare_fmt(p, s, z, f))
            del p, s, z
        y = torch.empty(1, n, dtype=torch.float32, device=dev)
        st = DecodeStep([GemvCall(preps[i % copies], n, k, x, y, f) for i in range(calls)])
        st.capture()
        ms = time_step(st, reps, 1)
        gbs = st.algorithmic_bytes() / (ms * 1e-3) / 1e9
        out[f"g{group}_{'bf16' if sbf else 'fp16'}_z{zb}"] = {
            "bits_per_weight": 4 + (16 + zb) / group, "us_per_call": round(ms * 1000 / calls, 2),
            "GB/s": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)}
        del st, preps
        torch.cuda.empty_cache()
    return out


def llama7b_layers(dev: str, layers: int = 6, reps: int = 5, fused: bool = False):
    """7B-shaped layers with 1 % outlier channels (x20 in W columns and x), bf16 x, M=1.

    ``layers`` distinct layers (6 x 106 MB, past the MALL) per step.  Unfused: seven
    w4_gemv calls per layer, each matrix with its own activation row.  Fused: the
    same-input matrices are concatenated along N (q|k|v 12288x4096, gate|up 22016x4096,
    each matrix keeping its own outlier columns) and share the first one's activation
    row, four calls per layer as in a real layer.
    """
    import torch

    import dequant_gemv_w4_amd as w4
    import synth
    from dequant_gemv_w4_amd.decode import DecodeStep, GemvCall

    groups = ((("q", "k", "v"), ("o",), ("gate", "up"), ("down",)) if fused
              else tuple((name,) for name in synth.MATRIX_ORDER))
    calls = []
    for layer in range(layers):
        for group in groups:
            parts = [synth.llama7b_layer_matrix(name, layer, dev) for name in group]
            W = torch.cat([w for w, _ in parts]) if len(parts) > 1 else parts[0][0]
            x = parts[0][1]
            n, k = W.shape
            p, s, z = w4.w4_quantize(W)
            calls.append(GemvCall(w4.w4_prepare(p, s, z), n, k, x,
                                  torch.empty(1, n, dtype=torch.float32, device=dev)))
            del W, parts, p, s, z
    st = DecodeStep(calls)
    st.capture()
    ms = time_step(st, reps, 1)
    us_layer = ms * 1000 / layers
    gbs = st.algorithmic_bytes() / (ms * 1e-3) / 1e9
    return {"layers_per_step": layers, "launches_per_layer": len(groups),
            "us_per_layer": round(us_layer, 2), "GB/s": round(gbs, 1),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "tokens_per_s_equiv_32_layers": round(1e6 / (32 * us_layer), 1)}


def prefill_gemm(prepared, dev: str, reps: int = 20, warmup: int = 10):
    import torch

    import dequant_gemv_w4_amd as w4
    import synth

    m, n, k = 4096, 28672, 8192
    X = synth.normal_activations(m, k, 40200, dev)
    Y = torch.empty(m, n, dtype=torch.float32, device=dev)
    ws = torch.empty(w4.w4_gemm_workspace_bytes(m, n, k), dtype=torch.uint8, device=dev)
    prep = prepared[(0, "gate")]
    for _ in range(warmup):   # the first calls after idle run slower (clock ramp)
        w4.w4_gemm(prep, n, k, X, Y=Y, workspace=ws)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        w4.w4_gemm(prep, n, k, X, Y=Y, workspace=ws)
    end.record()
    end.synchronize()
    ms = start.elapsed_time(end) / reps
    tflops = 2.0 * m * n * k / (ms * 1e-3) / 1e12
    # context on the same box: a dense bf16 product of the same shape through torch
    # (hipBLASLt): what a library GEMM on uncompressed 16-bit weights reaches
    Wt = torch.randn(k, n, device=dev, dtype=torch.float32).mul_(0.02).to(torch.bfloat16)
    for _ in range(warmup):
        Yd = torch.mm(X, Wt)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        Yd = torch.mm(X, Wt)
    end.record()
    end.synchronize()
    ms_d = start.elapsed_time(end) / reps
    del Wt, Yd
    return {"M": m, "N": n, "K": k, "ms": round(ms, 3), "TFLOP/s": round(tflops, 1),
            "mfma_util_vs_2.5PF_dense_bf16": round(tflops / BF16_DENSE_TFLOPS, 4),
            "dense_bf16_torch_matmul": {"ms": round(ms_d, 3),
                                        "TFLOP/s": round(2.0 * m * n * k / (ms_d * 1e-3) / 1e12, 1),
                                        "note": "torch.mm bf16 x bf16 -> bf16 (hipBLASLt), same "
                                                "shape, uncompressed weights"}}


def prefill_w8a8(dev: str, w4a16_ms: float | None, fmt: str = "fp8", reps: int = 20,
                 warmup: int = 10):
    """W8A8 (FP8 E4M3 or INT8) on the prefill shape: the same X and W draws as the W4A16 GEMM.

    W is quantized per output channel beforehand (untimed, as a checkpoint would be); the
    timed product is the per-token quantization of X plus the 8-bit GEMM, with the GEMM
    alone reported beside it.
    """
    import torch

    import dequant_gemv_w4_amd as w4
    import synth

    quant = w4.w4_fp8_quantize_rows if fmt == "fp8" else w4.w4_int8_quantize_rows
    gemm = w4.w4_fp8_gemm if fmt == "fp8" else w4.w4_int8_gemm
    m, n, k = 4096, 28672, 8192
    X = synth.normal_activations(m, k, 40200, dev)
    W = synth.normal_weights(n, k, synth.seed_for(4, "gate", 0), dev)
    wq, sw = quant(W)
    del W
    xq, sx = quant(X)
    Y = torch.empty(m, n, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        end.synchronize()
        return start.elapsed_time(end) / reps

    def full():
        quant(X, codes=xq, scales=sx)
        gemm(xq, sx, wq, sw, Y=Y)

    ms_full = timed(full)
    ms_gemm = timed(lambda: gemm(xq, sx, wq, sw, Y=Y))
    flops = 2.0 * m * n * k
    unit = "TFLOP/s" if fmt == "fp8" else "TOP/s"
    out = {"M": m, "N": n, "K": k, "ms": round(ms_full, 3),
           unit: round(flops / (ms_full * 1e-3) / 1e12, 1),
           "gemm_ms": round(ms_gemm, 3),
           "gemm_" + unit: round(flops / (ms_gemm * 1e-3) / 1e12, 1),
           f"mfma_util_vs_5P_dense_{fmt}": round(flops / (ms_gemm * 1e-3) / 1e12 / W8_DENSE_TOPS, 4)}
    if w4a16_ms:
        out["speedup_vs_w4a16_gemm"] = round(w4a16_ms / ms_full, 3)
    return out


def quantizer_rate(dev: str, reps: int = 3):
    import torch

    import dequant_gemv_w4_amd as w4
    import synth

    n, k = 28672, 8192
    W = synth.normal_weights(n, k, 40300, dev)
    p, s, z = w4.w4_quantize(W)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        w4.w4_quantize(W, packed=p, scales=s, zeros=z)
    end.record()
    end.synchronize()
    ms = start.elapsed_time(end) / reps
    nbytes = n * k * 4 + n * k // 2 + (n * k // 128) * 3
    return {"N": n, "K": k, "ms": round(ms, 3), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def _gemv_bytes(n: int, k: int, m: int, x_bytes: int) -> int:
    """Algorithmic bytes of one product: codes, fp16 scales, byte zeros, x, fp32 y."""
    return n * k // 2 + (n * k // 128) * 3 + m * k * x_bytes + m * n * 4


def cpu_baseline():
    """The oracle on the host cores, on a bounded sample of the workloads.

    Each configuration runs the oracle as it stands -- quantize_ref (binary32 emulation),
    then gemv_ref (fp64 dequantize-then-dot) -- on synthetic inputs drawn on the host:
    the page's 4096x4096 layer (binary32 x), one 7B-shaped layer and one 70B-shaped layer
    at M=1.  The 80-layer decode step is extrapolated as 80 x the 70B layer, and the
    prefill GEMM from 64 sampled rows of X (x 4096/64); both are labelled as such.
    ``value`` is the oracle's product rate on the 70B layer in the GPU metric's unit.
    """
    import numpy as np

    import oracle
    import synth

    def run(mats):
        tq = tg = 0.0
        nbytes = 0
        for W, x, x_bytes in mats():
            t0 = time.perf_counter()
            p, s, z = oracle.quantize_ref(W)
            t1 = time.perf_counter()
            oracle.gemv_ref(p, s, z, x)
            t2 = time.perf_counter()
            tq += t1 - t0
            tg += t2 - t1
            nbytes += _gemv_bytes(W.shape[0], W.shape[1], x.shape[0], x_bytes)
            del W, x, p, s, z
        return {"quantize_s": round(tq, 3), "gemv_s": round(tg, 3), "gemv_bytes": int(nbytes),
                "gemv_GB/s": round(nbytes / tg / 1e9, 4)}

    def page():
        w, x = synth.page_single_layer(4096, 4096)
        yield w, x, 4                      # binary32 x

    def layer7b():
        for name in synth.MATRIX_ORDER:
            W, x = synth.llama7b_layer_matrix(name, device="cpu")
            yield W.numpy(), x.float().numpy(), 2   # bf16 x

    def layer70b():
        for name in synth.MATRIX_ORDER:
            W, x = synth.llama70b_layer_matrix(name, device="cpu")
            yield W.numpy(), x.float().numpy(), 2

    res = {"page_single_layer_m1": run(page)}
    res["llama7b_layer_m1"] = run(layer7b)
    res["llama70b_layer_m1"] = run(layer70b)
    l70 = res["llama70b_layer_m1"]
    res["decode_step_m1_extrapolated"] = {
        "from": "80 x the 70B layer", "quantize_s": round(80 * l70["quantize_s"], 1),
        "gemv_s": round(80 * l70["gemv_s"], 1)}
    W, X = synth.prefill_operands(device="cpu")
    rows = np.random.default_rng(31).choice(X.shape[0], 64, replace=False)
    t0 = time.perf_counter()
    p, s, z = oracle.quantize_ref(W.numpy())
    t1 = time.perf_counter()
    oracle.gemv_ref(p, s, z, X[torch_index(rows)].float().numpy())
    t2 = time.perf_counter()
    res["prefill_gemm_extrapolated"] = {
        "from": "64 sampled rows of X x 4096/64", "quantize_s": round(t1 - t0, 3),
        "gemm_s": round((t2 - t1) * X.shape[0] / 64, 2),
        "TFLOP/s": round(2.0 * X.shape[0] * W.shape[0] * W.shape[1] / ((t2 - t1) * X.shape[0] / 64) / 1e12, 5)}
    del W, X, p, s, z

    threads = 1
    try:
        from threadpoolctl import threadpool_info
        threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:
        pass
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": l70["gemv_GB/s"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "oracle quantize_ref + gemv_ref (fp64) on the 4096x4096 page layer, one "
                      "7B-shaped and one 70B-shaped layer at M=1; value = gemv_ref rate on the "
                      "70B layer's algorithmic bytes; decode step and prefill GEMM extrapolated",
            "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "cpu_model": model,
            "configs": res}


def torch_index(rows):
    import torch
    return torch.from_numpy(rows)


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the method needs no "
                                   "inter-GPU communication and multi-GPU runs are not supported",
                          "n_gpus": args.gpus}))
        return 2

    import torch

    import dequant_gemv_w4_amd as w4
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w4.lib()
    if args.prefill_only:
        unfused = build_stack(1, dev, fused=False)
        print(json.dumps({"prefill_gemm": prefill_gemm(unfused, dev, reps=3, warmup=2)}), flush=True)
        return 0
    log(f"device {torch.cuda.get_device_name(0)}; building {args.layers} fused layers")
    prepared = build_stack(args.layers, dev, fused=True)

    if args.copy_calibration:
        src = torch.full((256 << 20,), 3, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    step = make_step(prepared, args.layers, 1, dev, fused=True)
    if not args.no_graph:
        step.capture()
        log("captured the step into a graph")
    step_ms: list = []
    ms = time_step(step, args.steps, args.warmup, per_step=step_ms)
    nbytes = step.algorithmic_bytes()
    gbs = nbytes / (ms * 1e-3) / 1e9
    launches = len(step.calls)
    log(f"step {ms:.3f} ms, {gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak)")

    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama70b-shaped decode step, batch 1: 80 layers x w4_gemv over "
                        "qkv 10240x8192 (q|k|v concatenated), o 8192x8192, gate_up 57344x8192 "
                        "(gate|up concatenated), down 8192x28672",
            "layers": args.layers,
            "gemv_launches_per_step": launches,
            "batch": 1,
            "resident_prepared_bytes": int(sum(t.numel() for t in prepared.values())),
            "algorithmic_bytes_per_step": int(nbytes),
            "graph_replay": not args.no_graph,
            "parallelism": "single GPU",
        },
        "tokens_per_s_equiv": round(1000.0 / ms, 2),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "step_ms_median_p10_p90": [round(percentile(step_ms, 0.5), 4),
                                   round(percentile(step_ms, 0.1), 4),
                                   round(percentile(step_ms, 0.9), 4)],
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": GEMV_STEP_TRAFFIC_BYTES_PER_LAUNCH,
            "traffic_unit": "bytes per launch (HBM, counter-measured)",
            "kernel": "w4_gemv (gemv_kernel, M=1 bf16 variants)",
            "per_launch": f"{nbytes / launches / 1e6:.2f} MB algorithmic in "
                          f"{ms * 1000 / launches:.2f} us average (step time / launches)",
        },
    }

    if not args.skip_extras:
        batches = {}
        for m in (4, 8, 16):
            st = make_step(prepared, args.layers, m, dev, fused=True)
            st.capture()
            msm = time_step(st, max(2, args.steps // 4), 1)
            batches[str(m)] = {"ms_per_step": round(msm, 3),
                               "GB/s": round(st.algorithmic_bytes() / (msm * 1e-3) / 1e9, 1),
                               "tokens_per_s": round(1000.0 * m / msm, 1)}
            del st
            log(f"M={m}: {msm:.3f} ms/step")
        result["batch_sweep_fused"] = batches
        result["per_shape_fused_m1"] = per_shape(prepared, args.layers, dev, fused=True, with_read=True)
        result["read_ceiling"] = read_ceiling(prepared, args.layers, dev, ms)
        log(f"read ceiling: {result['read_ceiling']}")
        del step, prepared
        torch.cuda.empty_cache()
        log("building the unfused stack")
        unfused = build_stack(args.layers, dev, fused=False)
        st = make_step(unfused, args.layers, 1, dev, fused=False)
        st.capture()
        msu = time_step(st, max(2, args.steps // 2), 2)
        result["unfused_step_m1"] = {
            "launches_per_step": len(st.calls), "ms_per_step": round(msu, 4),
            "GB/s": round(st.algorithmic_bytes() / (msu * 1e-3) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * st.algorithmic_bytes() / (msu * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        del st
        result["per_shape_m1"] = per_shape(unfused, args.layers, dev)
        log("per-shape done")
        result["prefill_gemm"] = prefill_gemm(unfused, dev)
        log(f"prefill GEMM: {result['prefill_gemm']}")
        result["prefill_w8a8_fp8"] = prefill_w8a8(dev, result["prefill_gemm"]["ms"], "fp8")
        log(f"prefill W8A8 FP8: {result['prefill_w8a8_fp8']}")
        result["prefill_w8a8_int8"] = prefill_w8a8(dev, result["prefill_gemm"]["ms"], "int8")
        log(f"prefill W8A8 INT8: {result['prefill_w8a8_int8']}")
        del unfused
        torch.cuda.empty_cache()
        result["quantizer"] = quantizer_rate(dev)
        result["page_single_layer_m1"] = page_layer(dev)
        log(f"page layer: {result['page_single_layer_m1']}")
        result["llama7b_layer_m1"] = llama7b_layers(dev)
        log(f"7B layers: {result['llama7b_layer_m1']}")
        result["llama7b_layer_fused_m1"] = llama7b_layers(dev, fused=True)
        log(f"7B layers, fused: {result['llama7b_layer_fused_m1']}")
        result["format_variants_m1"] = format_variants(dev)
        log(f"format variants: {result['format_variants_m1']}")

    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline()

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
