"""Seeded synthetic inputs for the PFA workloads (host side, numpy only).

This module is shared by the HIP path's tests/bench and by the fp64 oracle, so it
holds input recipes only and none of the method's arithmetic.

Recipe for Q, K, V of one layer: a numpy PCG64 stream seeded per (block, layer,
tensor) draws fp64 N(0, 1) values in C order of [B, heads, H, W, d]; they are
cast to fp32, multiplied in fp32 by the workload's scale (1/sqrt(d) for the
training-patch workload, 1 otherwise) and, for bf16 workloads, rounded to
nearest-even bf16. The rounded values are the ground truth for both sides.

Index matrix of the global workload: for token (y, x) of the H x W map, the k = 64
candidates are the 8x8 dilated neighbourhood (y + 4*(a-4), x + 4*(b-4)),
a, b = 0..7 (row-major over a then b; contains the token itself). Offsets that fall
outside the map are replaced, slot by slot, by uniform random tokens drawn from
a PCG64 stream, rejecting any token already in the row, so each row holds 64
distinct indices (not sorted).
"""

import numpy as np

from .workloads import Workload


def bf16_round_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to nearest-even bf16; returns the uint16 bit patterns."""
    bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


class Tensor:
    """One generated input tensor: ``device`` holds what the HIP path reads
    (fp32 values or bf16 bit patterns), ``exact`` the same values as fp32."""

    def __init__(self, device: np.ndarray, exact: np.ndarray, dtype: str):
        self.device = device
        self.exact = exact
        self.dtype = dtype


def draw(seed: int, shape, dtype: str, scale: float = 1.0) -> Tensor:
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape).astype(np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    if dtype == "f32":
        return Tensor(x, x, "f32")
    if dtype == "bf16":
        bits = bf16_round_bits(x)
        return Tensor(bits, bf16_bits_to_f32(bits), "bf16")
    raise ValueError(dtype)


def qkv(w: Workload, block: int, layer: int):
    """(Q, K, V) tensors of one layer, shape [B, heads, H, W, d]."""
    shape = (w.B, w.heads, w.H, w.W, w.d)
    return tuple(draw(w.qkv_seed(block, layer, t), shape, w.dtype, w.scale) for t in "qkv")


def global_index(w: Workload) -> np.ndarray:
    """[N, k] int32 candidate indices for the global workload (shared by all heads)."""
    H, W, k, dil = w.H, w.W, w.k_global, w.dilation
    side = int(round(k ** 0.5))
    assert side * side == k
    g = np.random.Generator(np.random.PCG64(w.index_seed))
    N = H * W
    offs = dil * (np.arange(side) - side // 2)
    out = np.empty((N, k), dtype=np.int32)
    for y in range(H):
        for x in range(W):
            ys = y + offs[:, None] + 0 * offs[None, :]
            xs = x + 0 * offs[:, None] + offs[None, :]
            inside = (ys >= 0) & (ys < H) & (xs >= 0) & (xs < W)
            row = np.where(inside, ys * W + xs, -1).reshape(-1)
            used = set(int(v) for v in row if v >= 0)
            for s in range(k):
                if row[s] < 0:
                    while True:
                        r = int(g.integers(0, N))
                        if r not in used:
                            break
                    used.add(r)
                    row[s] = r
            out[y * W + x] = row
    return out
