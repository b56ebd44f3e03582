"""Pins of the oracle's dense-rotation path (a QR-derived rotation for input dimensions the
Hadamard transform does not cover, VeloxQuant-MLX "Where the time actually went"): the
seeded rotation is orthogonal, and with the dense Hadamard-with-signs matrix in place of R
the dense path reproduces the pinned Hadamard path exactly."""

import numpy as np
import pytest

import workloads as wl
from oracle import encode as enc
from oracle import hadamard as hd
from oracle import ops


@pytest.mark.parametrize("K", [160, 4864 // 8, 4864])
def test_haar_rotation_is_orthogonal(K):
    R = wl.haar_rotation(K, 3).astype(np.float64)
    # float32 rounding of entries ~ 1/sqrt(K) leaves R R^T within a few ulp of I
    err = np.max(np.abs(R @ R.T - np.eye(K)))
    assert err < 2e-6, err
    x = np.random.default_rng(0).standard_normal((3, K))
    np.testing.assert_allclose(np.linalg.norm(ops.rotate_dense(x, R), axis=1),
                               np.linalg.norm(x, axis=1), rtol=2e-6)
    # a different seed gives a different rotation; the same seed the same bytes
    assert not np.array_equal(R, wl.haar_rotation(K, 4))
    assert np.array_equal(wl.haar_rotation(K, 3), wl.haar_rotation(K, 3))


@pytest.mark.parametrize("levels,group,K", [(8, 64, 512), (3, 16, 768), (16, 128, 1536)])
def test_dense_path_with_the_hadamard_matrix_is_the_hadamard_path(levels, group, K):
    g = wl.rng(995, levels, K)
    W = wl.student_rows(g, 20, K).astype(np.float64)
    R = hd.rotation_matrix(K, 6)
    a, b = enc.encode(W, levels, group, 6), enc.encode_dense(W, R, levels, group)
    mism = a.idx != b.idx
    assert not np.any(mism & ~enc.near_threshold(a.u, levels, 1e-6))
    assert np.array_equal(a.scales, b.scales) or np.all(
        enc.fp16_bits(a.r * (1 - 1e-9)) != enc.fp16_bits(a.r * (1 + 1e-9)))
    x = g.standard_normal(K)
    np.testing.assert_allclose(ops.qmv_dense(a.codes, a.scales, levels, group, K, R, x),
                               ops.qmv(a.codes, a.scales, levels, group, K, 6, x), rtol=1e-12,
                               atol=1e-12)


def test_dense_encode_of_a_4864_wide_layer():
    # K = 4864 = 19 * 256 has no Hadamard matrix here; the dense path encodes it, with the
    # per-group normalization intact: mean(u^2) = 1 in every group
    K, levels, group = 4864, 8, 128
    W = wl.student_rows(wl.rng(996, 0), 6, K).astype(np.float64)
    R = wl.haar_rotation(K, 1)
    e = enc.encode_dense(W, R, levels, group)
    G = e.u.reshape(6, K // group, group)
    np.testing.assert_allclose(np.mean(G * G, axis=-1), 1.0, rtol=1e-12)
    with pytest.raises(ValueError):
        hd.split_dim(K)
