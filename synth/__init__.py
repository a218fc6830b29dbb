"""Seeded synthetic inputs for the W4A16 hot path.

This module only draws numbers.  It holds none of the quantization or
dot-product arithmetic, so both the CPU oracle and the HIP path can take their
inputs from it without sharing any part of the method.

Recipes (stand-ins for the pages' Llama-shaped workloads; no model weights or
datasets are used):

* ``xorshift_uniform`` -- the 64-bit xorshift stream of the "Weight
  quantization" page (section "Code", its ``main`` routine): shifts 13/7/17,
  seed 0x9E3779B97F4A7C15, each draw mapped to f32 in [-1, 1) by taking the
  top 53 bits, converting to f32, dividing by 2^53 and computing ``2u - 1`` in
  f32.  The 4096x4096 single-layer workload draws W row-major (scaled by 0.02
  in f32) and then x.
* ``normal_weights`` / ``normal_activations`` -- N(0, 0.02) f32 weights and
  N(0, 1) activations rounded to bf16 (round-to-nearest-even), drawn with a
  torch generator on the requested device.
* ``outlier_channels`` -- about 1 % of the input channels (``round(0.01*K)``)
  picked by a seeded permutation; weights and activations of those channels are
  scaled by 20 in f32 before any rounding.
"""

from __future__ import annotations

import numpy as np

XORSHIFT_SEED = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1

# Model shapes the workloads use (out_features N, in_features K).
LLAMA7B_SHAPES = {
    "q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
    "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008),
}
LLAMA70B_SHAPES = {
    "q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
    "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672),
}
MATRIX_ORDER = ("q", "k", "v", "o", "gate", "up", "down")
# same-input matrices concatenated along N (one launch per group)
LLAMA70B_FUSED_SHAPES = {"qkv": (10240, 8192), "o": (8192, 8192), "gate_up": (57344, 8192),
                         "down": (8192, 28672)}
FUSED_ORDER = ("qkv", "o", "gate_up", "down")
FUSED_PARTS = {"qkv": ("q", "k", "v"), "o": ("o",), "gate_up": ("gate", "up"), "down": ("down",)}


def seed_for(workload: int, matrix: str, layer: int = 0) -> int:
    """Seed of one weight matrix: 20260000 + 100*workload + matrix index + 1000*layer."""
    return 20260000 + 100 * workload + MATRIX_ORDER.index(matrix) + 1000 * layer


# --------------------------------------------------------------------------
# xorshift64 stream
# --------------------------------------------------------------------------

def _xorshift_step(s: int) -> int:
    s ^= (s << 13) & _MASK64
    s ^= s >> 7
    s ^= (s << 17) & _MASK64
    return s


def _step_matrix_columns() -> list[int]:
    """Images of the 64 unit vectors under one xorshift step (the map is linear over GF(2))."""
    return [_xorshift_step(1 << b) for b in range(64)]


def _compose(a_cols: list[int], b_cols: list[int]) -> list[int]:
    """Columns of the map A∘B (apply B, then A)."""
    out = []
    for c in b_cols:
        r = 0
        b = 0
        while c:
            if c & 1:
                r ^= a_cols[b]
            c >>= 1
            b += 1
        out.append(r)
    return out


def _byte_tables(cols: list[int]) -> np.ndarray:
    """8 lookup tables of 256 entries: the map applied to each byte value at each byte position."""
    tabs = np.zeros((8, 256), dtype=np.uint64)
    for j in range(8):
        for v in range(256):
            r = 0
            for b in range(8):
                if (v >> b) & 1:
                    r ^= cols[8 * j + b]
            tabs[j, v] = r
    return tabs


def _apply(tabs: np.ndarray, states: np.ndarray) -> np.ndarray:
    out = np.zeros_like(states)
    for j in range(8):
        idx = ((states >> np.uint64(8 * j)) & np.uint64(0xFF)).astype(np.intp)
        out ^= tabs[j][idx]
    return out


def xorshift_states(count: int, seed: int = XORSHIFT_SEED) -> np.ndarray:
    """The first ``count`` states of the stream; state i is the state after i+1 steps."""
    if count <= 0:
        return np.zeros(0, dtype=np.uint64)
    block = min(count, 4096)
    first = np.empty(block, dtype=np.uint64)
    s = seed
    for i in range(block):
        s = _xorshift_step(s)
        first[i] = s
    out = np.empty(count, dtype=np.uint64)
    out[:block] = first
    have = block
    # jump map for `have` steps, built by repeated composition
    cols1 = _step_matrix_columns()
    jump = [1 << b for b in range(64)]  # identity
    p, e, n = cols1, 1, have
    while n:  # jump = step^have by square-and-multiply
        if n & 1:
            jump = _compose(p, jump)
        n >>= 1
        if n:
            p = _compose(p, p)
        e *= 2
    while have < count:
        take = min(have, count - have)
        tabs = _byte_tables(jump)
        out[have:have + take] = _apply(tabs, out[:take])
        have += take
        jump = _compose(jump, jump)
    return out


def xorshift_uniform(count: int, seed: int = XORSHIFT_SEED) -> np.ndarray:
    """f32 draws in [-1, 1): ((s >> 11) as f32) / 2^53 * 2 - 1, every step in f32."""
    s = xorshift_states(count, seed)
    top = (s >> np.uint64(11)).astype(np.float64)       # exact: below 2^53
    u = top.astype(np.float32)                          # one rounding, nearest-even
    u = u / np.float32(2.0 ** 53)                       # power of two: exact
    return (u * np.float32(2.0)) - np.float32(1.0)      # two separate f32 roundings


def page_single_layer(n: int = 4096, k: int = 4096) -> tuple[np.ndarray, np.ndarray]:
    """W [n, k] = 0.02 * U(-1, 1) in f32 (row-major draws), then x [1, k] = U(-1, 1)."""
    r = xorshift_uniform(n * k + k)
    w = (np.float32(0.02) * r[: n * k]).reshape(n, k)
    x = r[n * k:].reshape(1, k).copy()
    return w, x


# --------------------------------------------------------------------------
# Gaussian Llama-shaped layers (torch, any device)
# --------------------------------------------------------------------------

def _gen(seed: int, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_weights(n: int, k: int, seed: int, device="cpu", std: float = 0.02):
    """W [n, k] f32 ~ N(0, std)."""
    import torch
    g = _gen(seed, device)
    w = torch.randn(n, k, generator=g, device=device, dtype=torch.float32)
    return w.mul_(std)


def normal_activations(m: int, k: int, seed: int, device="cpu", dtype=None):
    """x [m, k] ~ N(0, 1) in f32, rounded to ``dtype`` (default bf16) if given."""
    import torch
    g = _gen(seed, device)
    x = torch.randn(m, k, generator=g, device=device, dtype=torch.float32)
    if dtype is None:
        dtype = torch.bfloat16
    return x.to(dtype)


def outlier_channels(k: int, seed: int, device="cpu", frac: float = 0.01):
    """round(frac*k) input channels chosen by a seeded permutation of range(k)."""
    import torch
    g = _gen(seed + 7, "cpu")
    cnt = int(round(frac * k))
    ch = torch.randperm(k, generator=g)[:cnt]
    return ch.to(device)


def llama7b_layer_matrix(matrix: str, layer: int = 0, device="cpu", m: int = 1):
    """One matrix of the 7B-shaped layer with outlier channels, plus its bf16 activations.

    Returns (W f32 [N, K], x bf16 [m, K]).  The selected channels are scaled by 20 in
    both W (columns) and x (f32, before the bf16 rounding).
    """
    import torch
    n, k = LLAMA7B_SHAPES[matrix]
    seed = seed_for(2, matrix, layer)
    w = normal_weights(n, k, seed, device)
    gx = _gen(seed + 50, device)
    x = torch.randn(m, k, generator=gx, device=device, dtype=torch.float32)
    ch = outlier_channels(k, seed, device)
    w[:, ch] *= 20.0
    x[:, ch] *= 20.0
    return w, x.to(torch.bfloat16)


def llama70b_layer_matrix(matrix: str, layer: int = 0, device="cpu", m: int = 1):
    """One matrix of the 70B-shaped GQA layer (no outliers) with bf16 activations."""
    n, k = LLAMA70B_SHAPES[matrix]
    seed = seed_for(3, matrix, layer)
    w = normal_weights(n, k, seed, device)
    x = normal_activations(m, k, seed + 50, device)
    return w, x


def prefill_operands(device="cpu", m: int = 4096, n: int = 28672, k: int = 8192):
    """Prefill GEMM operands: W [n, k] ~ N(0, 0.02) f32 and X [m, k] ~ N(0, 1) bf16."""
    seed = seed_for(5, "gate")
    w = normal_weights(n, k, seed, device)
    x = normal_activations(m, k, seed + 50, device)
    return w, x


def page_error_matrix(seed: int = 11, rows: int = 256, cols: int = 1024) -> np.ndarray:
    """Seeded 256 x 1024 test matrix of page "Quantization", section "Code" (fp64).

    Row r is Gaussian with standard deviation 0.02 * exp(g_r), g_r ~ N(0, 0.5);
    then eight entries become +-0.6 outliers.  Draws come from Python's seeded
    Mersenne-Twister generator in the page's order: per row the deviation draw and
    the row's values; per outlier its sign, its row and its column (the page's
    one-line assignment evaluates the value before the subscripts).
    """
    import math
    import random

    rng = random.Random(seed)
    w = np.empty((rows, cols), dtype=np.float64)
    for r in range(rows):
        sd = 0.02 * math.exp(rng.gauss(0.0, 0.5))
        w[r] = [rng.gauss(0.0, sd) for _ in range(cols)]
    for _ in range(8):
        sign = rng.choice((-1, 1))
        r = rng.randrange(rows)
        c = rng.randrange(cols)
        w[r, c] = sign * 0.6
    return w



# --------------------------------------------------------------------------
# Sparse groups and wide-range activations (edge cases of the products)
# --------------------------------------------------------------------------

def sparse_group_weights(n: int, k: int, seed: int, group: int = 128):
    """W [n, k] f32 in which every group of ``group`` inputs has 1-3 non-zero weights at
    positions shared by all rows (the rest exact 0.0), one of them negative and one
    positive where there are two or more, so that the zero point of most groups is neither
    0 nor 15 and most codes equal it.  Returns (W, positions [k] bool).
    """
    rng = np.random.default_rng(seed)
    pos = np.zeros(k, dtype=bool)
    for g in range(k // group):
        cnt = int(rng.integers(1, 4))
        pos[g * group + rng.choice(group, cnt, replace=False)] = True
    w = np.zeros((n, k), dtype=np.float32)
    idx = np.flatnonzero(pos)
    mag = (0.02 * (0.5 + rng.random((n, idx.size)))).astype(np.float32)
    sign = np.where(rng.random((n, idx.size)) < 0.5, -1.0, 1.0).astype(np.float32)
    # the first non-zero of each group negative, the second positive (when present)
    g_of = idx // group
    first = np.r_[True, g_of[1:] != g_of[:-1]]
    second = np.r_[False, first[:-1] & (g_of[1:] == g_of[:-1])]
    sign[:, first] = -1.0
    sign[:, second] = 1.0
    w[:, idx] = mag * sign
    return w, pos


def sparse_group_activations(m: int, positions: np.ndarray, seed: int, small: float = 1e-2,
                             large: float = 3.0):
    """x [m, k] f32: about ``small`` in magnitude at ``positions``, about ``large`` elsewhere,
    random signs."""
    rng = np.random.default_rng(seed)
    k = positions.size
    mag = np.where(positions, small, large) * (1.0 + 0.1 * rng.standard_normal((m, k)))
    sign = np.where(rng.random((m, k)) < 0.5, -1.0, 1.0)
    return (mag * sign).astype(np.float32)


def wide_range_activations(m: int, k: int, seed: int, span_log2: int = 40):
    """x [m, k] f32 ~ N(0, 1) in which every fourth 32-input slice also holds one value
    2^(span/2) times larger and one 2^(span/2) times smaller than the rest, so that a slice
    spans about 2^span in magnitude."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k))
    half = 2.0 ** (span_log2 // 2)
    for s in range(0, k // 32, 4):
        a, b = rng.choice(32, 2, replace=False)
        x[:, 32 * s + a] *= half
        x[:, 32 * s + b] /= half
    return x.astype(np.float32)
