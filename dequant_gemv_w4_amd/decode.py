"""A decode step: every quantized matrix of a model multiplied once by its activation rows.

Decode reads each weight once per generated token, so the step time is bounded
below by (weight bytes) / (HBM bandwidth) (page "Weight quantization", sections
"Complexity and constants" and "Efficiency"; page "Quantization" › "The idea in
one minute").  ``DecodeStep`` issues the w4_gemv calls of such a step back to
back on one stream and can capture them once into a graph, so replaying a step
costs a single launch from the host.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

from . import W4_BF16, W4_F32, W4Error, lib


@dataclass
class GemvCall:
    prepared: object   # uint8 tensor from w4_prepare (or w4_prepare_fmt)
    n: int
    k: int
    x: object          # [M, K] bf16 or f32 tensor
    y: object          # [M, N] f32 or bf16 tensor
    fmt: object = None  # W4Format of the prepared layout; None: the canonical format

    def algorithmic_bytes(self) -> int:
        """Bytes the method must move: codes, scales and zeros as the format stores them
        (canonical: fp16 scales and byte zeros per 128 inputs), activations, outputs."""
        m = self.x.shape[0]
        group, zero_bits = (128, 8) if self.fmt is None else (self.fmt.group, self.fmt.zero_bits)
        groups = self.n * self.k // group
        return (self.n * self.k // 2 + groups * 2 + (groups * zero_bits + 7) // 8
                + m * self.k * self.x.element_size() + m * self.n * self.y.element_size())


class DecodeStep:
    def __init__(self, calls: list[GemvCall]):
        import torch
        self.calls = calls
        self._graph = None
        L = lib()
        self._args = []
        for c in calls:
            if c.x.shape[1] != c.k or c.y.shape != (c.x.shape[0], c.n):
                raise ValueError("inconsistent GEMV shapes")
            xt = W4_F32 if c.x.dtype == torch.float32 else W4_BF16
            yt = W4_F32 if c.y.dtype == torch.float32 else W4_BF16
            head = (ctypes.c_void_p(c.prepared.data_ptr()), c.n, c.k)
            tail = (ctypes.c_void_p(c.x.data_ptr()), xt, c.x.shape[0],
                    ctypes.c_void_p(c.y.data_ptr()), yt)
            if c.fmt is None:
                self._args.append((L.w4_gemv, "w4_gemv", head + tail))
            else:
                self._args.append((L.w4_gemv_fmt, "w4_gemv_fmt", head + (ctypes.byref(c.fmt),) + tail))

    def algorithmic_bytes(self) -> int:
        return sum(c.algorithmic_bytes() for c in self.calls)

    def run_eager(self) -> None:
        import torch
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for fn, name, a in self._args:
            st = fn(*a, s)
            if st != 0:
                raise W4Error(st, name)

    def capture(self) -> None:
        """Record the whole step once into a graph (replayed by run())."""
        import torch
        self.run_eager()                      # warm caches and the device check outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_eager()
        torch.cuda.synchronize()
        self._graph = g

    def run(self) -> None:
        if self._graph is not None:
            self._graph.replay()
        else:
            self.run_eager()
