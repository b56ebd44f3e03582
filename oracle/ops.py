"""The fused quantized linear layers, by their definitions, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: turboquant-mlx "How it works", section "Running a quantized layer": the layer
rotates its input with the same orthonormal rotation and multiplies by the packed weights,
y_i = sum_g scale_{i,g} sum_{j in g} c[idx_ij] x'_j with x' = R x, because
(R w) . (R x) = w . x. The kernel table in that section names the Mixture-of-Experts forms:
  gather_qmv        one token: each routed expert reads the same input;
  multi_gather_qmv  a different input per (input, expert) pair;
  gather_qmm        a large batch of rows sorted by expert (a batched gather-GEMM).
Each is checked on the page against a reference dequantize-and-multiply; these functions
are exactly that: dequantize (``encode.dequant``), then multiply in fp64.

Readings: y rows of gather_qmm are in the sorted-row order of the caller; row m belongs to
the expert e with offsets[e] <= m < offsets[e + 1] and reads input row row_token[m].
"""

import numpy as np

from . import encode as enc
from . import hadamard as hd


def qmv(codes, scales, levels, group, K, seed, x):
    """y = w'_hat . (R x) for every row; x has shape [K] or [B][K] (B inputs)."""
    Wq = enc.dequant(codes, scales, levels, group, K)
    xr = hd.rotate(np.asarray(x, dtype=np.float64), seed)
    return xr @ Wq.T


def qmv_unrotated(codes, scales, levels, group, K, seed, x):
    """The same product taken in the original basis: (R^T w'_hat) . x."""
    W = enc.dequant_unrotated(codes, scales, levels, group, K, seed)
    return np.asarray(x, dtype=np.float64) @ W.T


def gather_qmv(codes, scales, levels, group, K, seed, ids, x):
    """y[k] = W_{ids[k]} R x for k = 0..len(ids)-1; codes/scales are [E][N][...]."""
    return np.stack([qmv(codes[e], scales[e], levels, group, K, seed, x) for e in ids])


def multi_gather_qmv(codes, scales, levels, group, K, seed, ids, X):
    """y[p] = W_{ids[p]} R X[p] for every pair p."""
    X = np.asarray(X, dtype=np.float64)
    return np.stack([qmv(codes[e], scales[e], levels, group, K, seed, X[p])
                     for p, e in enumerate(ids)])


def gather_qmm(codes, scales, levels, group, K, seed, X, row_token, offsets):
    """y[m] = W_e R X[row_token[m]] for offsets[e] <= m < offsets[e+1]."""
    X = np.asarray(X, dtype=np.float64)
    E = len(offsets) - 1
    N = codes.shape[1]
    M = int(offsets[-1])
    y = np.zeros((M, N))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = qmv(codes[e], scales[e], levels, group, K, seed, X[row_token[a:b]])
    return y


def row_bound(codes, scales, levels, group, K, x, rel=2e-3):
    """Per-row output tolerance rel * ||x|| * ||w'_hat_i|| (x as given; ||R x|| = ||x||)."""
    Wq = enc.dequant(codes, scales, levels, group, K)
    xn = np.linalg.norm(np.asarray(x, dtype=np.float64), axis=-1)
    return rel * np.multiply.outer(xn, np.linalg.norm(Wq, axis=-1))


def qmv_dense(codes, scales, levels, group, K, R, x):
    """y = w'_hat . (R x) with a dense orthogonal rotation R [K][K] (VeloxQuant-MLX's
    QR-derived rotation; "Running a quantized layer" of turboquant-mlx: rotate the input,
    multiply by the decoded rotated weights)."""
    Wq = enc.dequant(codes, scales, levels, group, K)
    xr = np.asarray(x, dtype=np.float64) @ np.asarray(R, dtype=np.float64).T
    return xr @ Wq.T


def rotate_dense(X, R):
    """Rows of X mapped to R x."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(R, dtype=np.float64).T
