"""Pins of the oracle's qmv family.

* qmv in the rotated basis equals the product with the de-rotated dequantized weights in
  the original basis (the identity the layer relies on: turboquant-mlx "How it works",
  "Running a quantized layer").
* A pure-Python brute force on tiny shapes -- indices read back bit by bit, rotation
  built entry by entry from the closed form (-1)^popcount(i & j) and the signs -- equals
  qmv: this is the "reference dequantize-and-multiply" the page tests its kernels against.
* The gather forms equal per-expert / per-pair qmv by construction of their inputs.
* Quantization error of y against the unquantized W x is of the size the codebook's
  distortion predicts.
"""

import math

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import encode as enc
from oracle import hadamard as hd
from oracle import ops


def brute_qmv(codes, scales, levels, group, K, seed, x):
    """Pure-Python loops; shares only the codebook values and signs with the oracle."""
    c = cb.centroids(levels)
    s = hd.signs(seed, K)
    N = codes.shape[0]
    # x' = H (s * x) / sqrt(K) with H[i][j] = (-1)^popcount(i & j) (K a power of two)
    xr = []
    for i in range(K):
        acc = 0.0
        for j in range(K):
            h = -1.0 if bin(i & j).count("1") % 2 else 1.0
            acc += h * s[j] * float(x[j])
        xr.append(acc / math.sqrt(K))
    y = []
    for r in range(N):
        words = [int(w) for w in codes[r]]
        total = 0.0
        for j in range(K):
            if levels == 3:
                w = words[j // 20]
                for _ in range(j % 20):
                    w //= 3
                idx = w % 3
            else:
                b = int(math.log2(levels))
                idx = 0
                for q in range(b):
                    p = b * j + q
                    idx |= ((words[p // 32] >> (p % 32)) & 1) << q
            sc = float(np.uint16(scales[r, j // group]).view(np.float16))
            total += c[idx] * sc * xr[j]
        y.append(total)
    return np.array(y)


@pytest.mark.parametrize("levels,group,K", [(16, 16, 32), (8, 32, 64), (4, 16, 64), (3, 16, 64)])
def test_brute_force_tiny(levels, group, K):
    rng = np.random.default_rng(levels + K)
    W = rng.standard_t(4, (5, K))
    x = rng.standard_normal(K)
    e = enc.encode(W, levels, group, seed=9)
    want = brute_qmv(e.codes, e.scales, levels, group, K, 9, x)
    got = ops.qmv(e.codes, e.scales, levels, group, K, 9, x)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("levels,group,K", [(16, 64, 512), (8, 128, 768), (4, 64, 1536),
                                            (3, 16, 640)])
def test_rotated_equals_unrotated(levels, group, K):
    rng = np.random.default_rng(K)
    W = rng.standard_t(4, (16, K))
    x = rng.standard_normal((3, K))
    e = enc.encode(W, levels, group, seed=5)
    a = ops.qmv(e.codes, e.scales, levels, group, K, 5, x)
    b = ops.qmv_unrotated(e.codes, e.scales, levels, group, K, 5, x)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)


def test_quantization_error_size():
    rng = np.random.default_rng(0)
    K, N = 1024, 256
    W = rng.standard_normal((N, K))
    x = rng.standard_normal(K)
    exact = W @ x
    for levels, group in ((16, 64), (8, 64), (4, 64), (3, 16)):
        e = enc.encode(W, levels, group, seed=0)
        y = ops.qmv(e.codes, e.scales, levels, group, K, 0, x)
        rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
        # error of a product with i.i.d. quantization noise: ~ sqrt(D)
        D = cb.distortion(levels)
        assert 0.5 * math.sqrt(D) < rel < 1.5 * math.sqrt(D), (levels, rel, D)


def make_experts(rng, E, N, K, levels, group, seed):
    codes, scales = [], []
    for _ in range(E):
        e = enc.encode(rng.standard_t(4, (N, K)), levels, group, seed)
        codes.append(e.codes)
        scales.append(e.scales)
    return np.stack(codes), np.stack(scales)


def test_gather_forms():
    rng = np.random.default_rng(1)
    E, N, K, L, g, seed = 6, 12, 256, 8, 32, 4
    codes, scales = make_experts(rng, E, N, K, L, g, seed)
    x = rng.standard_normal(K)
    ids = [4, 0, 5]
    y = ops.gather_qmv(codes, scales, L, g, K, seed, ids, x)
    for k, e in enumerate(ids):
        np.testing.assert_allclose(y[k], ops.qmv(codes[e], scales[e], L, g, K, seed, x))
    X = rng.standard_normal((5, K))
    pids = [2, 2, 0, 5, 1]
    ym = ops.multi_gather_qmv(codes, scales, L, g, K, seed, pids, X)
    for p, e in enumerate(pids):
        np.testing.assert_allclose(ym[p], ops.qmv(codes[e], scales[e], L, g, K, seed, X[p]))
    # gather_qmm: rows sorted by expert, offsets, token gather
    T = 4
    Xt = rng.standard_normal((T, K))
    row_token = np.array([1, 3, 0, 0, 2, 1, 3])
    offsets = np.array([0, 2, 2, 4, 5, 7, 7])
    yq = ops.gather_qmm(codes, scales, L, g, K, seed, Xt, row_token, offsets)
    for m in range(7):
        e = int(np.searchsorted(offsets, m, side="right") - 1)
        np.testing.assert_allclose(yq[m], ops.qmv(codes[e], scales[e], L, g, K, seed,
                                                  Xt[row_token[m]]))


def test_row_bound_shape():
    rng = np.random.default_rng(2)
    e = enc.encode(rng.standard_normal((4, 64)), 16, 16, 0)
    x = rng.standard_normal(64)
    b = ops.row_bound(e.codes, e.scales, 16, 16, 64, x)
    assert b.shape == (4,)
    Wq = enc.dequant(e.codes, e.scales, 16, 16, 64)
    np.testing.assert_allclose(b, 2e-3 * np.linalg.norm(x) * np.linalg.norm(Wq, axis=1))
