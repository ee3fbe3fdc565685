"""Hadamard matrix, fast Walsh-Hadamard transform and vector norm in fp32.

PolyKV explainer, section 2.B (value rotation): each V vector is rotated by
a fast Walsh-Hadamard transform before scalar quantisation.  The page gives no
normalisation, ordering or sign convention.  Reading used here:

* H is the unnormalised Sylvester matrix in natural order:
  H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]], so H[i][j] = (-1)^popcount(i & j),
  H is symmetric and H @ H = d * I.
* FWHT(x) = H @ x, computed by log2(d) butterfly stages with the half-width h
  ascending (1, 2, 4, ...); at each stage the pair (z_i, z_{i+h}), i & h == 0,
  becomes (z_i + z_{i+h}, z_i - z_{i+h}).  Every add/sub is one fp32 rounding.
* No random sign flips (the page mentions none).

The vector norm is the plain L2 norm of the fp32 vector, with squares summed
by a fixed halving tree (h = d/2, d/4, ..., 1: s_i <- s_i + s_{i+h} for i < h),
then a correctly rounded square root.  Fixing the order makes the fp32 result
a single defined value.
"""
from __future__ import annotations

import numpy as np


def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), int64 entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """H @ x along the last axis, fp32 butterflies with ascending half-width."""
    z = np.array(x, dtype=np.float32, copy=True)
    d = z.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("last axis must be a power of two")
    lead = z.shape[:-1]
    h = 1
    while h < d:
        zz = z.reshape(lead + (d // (2 * h), 2, h))
        a = zz[..., 0, :]
        b = zz[..., 1, :]
        z = np.stack([a + b, a - b], axis=-2).reshape(lead + (d,))
        h *= 2
    return z


def sumsq_tree_f32(x: np.ndarray) -> np.ndarray:
    """Sum of squares along the last axis in the fixed halving-tree order, fp32."""
    s = np.asarray(x, dtype=np.float32)
    s = s * s
    h = s.shape[-1] // 2
    while h >= 1:
        s = s[..., :h] + s[..., h:2 * h]
        h //= 2
    return s[..., 0]


def norm_f32(x: np.ndarray) -> np.ndarray:
    """L2 norm along the last axis: correctly rounded sqrt of the tree sum of squares."""
    return np.sqrt(sumsq_tree_f32(x)).astype(np.float32)
