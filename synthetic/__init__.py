"""Seeded synthetic int8 matrices shared by the tests, the bench and smoke().

This module holds no GEMM arithmetic: it only draws uniform int8 values.  Both
the GPU path and the CPU oracle receive the bytes it produces, so neither side
draws random numbers of its own.

Generator: SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014), used counter-style.  Output number n
(n = 1, 2, ...) of a stream started at state s0 is

    z = s0 + n * 0x9E3779B97F4A7C15          (mod 2**64)
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9  (mod 2**64)
    z = (z ^ (z >> 27)) * 0x94D049BB133111EB  (mod 2**64)
    z =  z ^ (z >> 31)

which is exactly the sequential generator's n-th output.  Element idx of a
logical matrix (row-major index, independent of the storage layout) takes the
low byte of output idx + 1, read as a signed int8, so every value in
[-128, 127] is equally likely and both ends are reachable.  The stream start is
s0 = seed * 256 + tag (tag 1 for A, 2 for B), so seed 0 / tag 0 is the
reference stream whose first outputs are published with the generator.
"""
from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
MUL1 = np.uint64(0xBF58476D1CE4E5B9)
MUL2 = np.uint64(0x94D049BB133111EB)

TAG_A = 1
TAG_B = 2

_CHUNK = 1 << 22  # elements per vectorised chunk (32 MiB of uint64 temporaries)


def stream_start(seed: int, tag: int) -> int:
    return (int(seed) * 256 + int(tag)) % (1 << 64)


def splitmix64_outputs(s0: int, first: int, count: int) -> np.ndarray:
    """Outputs number first+1 .. first+count of the stream started at s0."""
    with np.errstate(over="ignore"):
        n = np.arange(first + 1, first + count + 1, dtype=np.uint64)
        z = np.uint64(s0) + n * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * MUL1
        z = (z ^ (z >> np.uint64(27))) * MUL2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform_int8(rows: int, cols: int, seed: int, tag: int) -> np.ndarray:
    """Logical rows x cols int8 matrix (C-contiguous), uniform in [-128, 127]."""
    total = int(rows) * int(cols)
    out = np.empty(total, dtype=np.int8)
    s0 = stream_start(seed, tag)
    for start in range(0, total, _CHUNK):
        cnt = min(_CHUNK, total - start)
        z = splitmix64_outputs(s0, start, cnt)
        out[start:start + cnt] = (z & np.uint64(0xFF)).astype(np.uint8).view(np.int8)
    return out.reshape(rows, cols)


def gemm_inputs(M: int, N: int, K: int, seed: int):
    """Logical A (M x K) and B (K x N) for one seed."""
    return uniform_int8(M, K, seed, TAG_A), uniform_int8(K, N, seed, TAG_B)


def store_b(B_logical: np.ndarray, b_col_major: bool) -> np.ndarray:
    """Storage of the logical K x N matrix B: itself (row-major) or its
    transpose made contiguous (column-major, i.e. N x K with K contiguous)."""
    return np.ascontiguousarray(B_logical.T) if b_col_major else np.ascontiguousarray(B_logical)


def freivalds_vectors(N: int, count: int, seed: int) -> np.ndarray:
    """count x N int64 vectors with entries in [-8, 7] (tag 3) for the
    randomised product check C x == A (B x)."""
    v = uniform_int8(count, N, seed, 3).astype(np.int64)
    return v >> 4


def conv_inputs(N: int, H: int, W: int, C: int, K: int, R: int, S: int, seed: int):
    """(x, w) for a convolution: x int8 N x H x W x C (NHWC, stream tag 4) and
    w int8 K x R x S x C (KRSC, tag 5), uniform over all 256 values, element
    index = the row-major index of each array."""
    x = uniform_int8(N * H * W, C, seed, 4).reshape(N, H, W, C)
    w = uniform_int8(K * R * S, C, seed, 5).reshape(K, R, S, C)
    return x, w
