"""Pins of the oracle's encode step.

* fp16 scale rounding equals a brute-force nearest search over every finite fp16 value
  (ties to the even significand), saturating at 65504.
* Normalized groups have mean(u^2) = 1; the snap equals a brute-force nearest centroid
  away from thresholds.
* Distortion: on rotated heavy-tailed rows, E[(u - c[idx])^2] is within a few % of the
  distortion of i.i.d. Gaussian groups of the same size (sampled, brute-force nearest
  centroid): the rotation makes the rows Gaussian-like. For groups of 64 and more this is
  also close to the codebook's N(0,1) distortion.
* Power-of-two scaling of W scales the stored fp16 scales exactly and leaves codes alone.
* Encoding row chunks gives the same bytes as encoding the whole matrix (the streaming
  converter's output is byte-identical to the in-memory one: turboquant-mlx "How it
  works", "Two converters").
* Zero rows encode to scale 0 and dequantize to exactly 0.
"""

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import encode as enc
from oracle import hadamard as hd


def all_finite_fp16():
    bits = np.arange(0, 0x7C00, dtype=np.uint16)  # +0 .. largest finite
    return bits, bits.view(np.float16).astype(np.float64)


def brute_fp16(r):
    bits, vals = all_finite_fp16()
    out = []
    for v in r:
        if v >= 65504.0:
            out.append(0x7BFF)
            continue
        d = np.abs(vals - v)
        k = np.flatnonzero(d == d.min())
        if len(k) == 2:  # tie: even significand
            k = k[np.argmin(bits[k] & 1)]
        out.append(int(bits[int(np.ravel(k)[0])]))
    return np.array(out, dtype=np.uint16)


def test_fp16_scale_rounding():
    rng = np.random.default_rng(0)
    _, vals = all_finite_fp16()
    mids = (vals[1:200] + vals[:199]) / 2  # exact midpoints: ties
    r = np.concatenate([
        rng.lognormal(0, 3, 3000), rng.uniform(0, 1e-4, 500), mids,
        [0.0, 5.96e-8, 65504.0, 65519.9, 65520.0, 1e9],
    ])
    np.testing.assert_array_equal(enc.fp16_bits(r), brute_fp16(r))


def student_rows(rng, n, K):
    W = rng.standard_t(4, (n, K)) * np.exp(rng.normal(0, 0.5, (n, 1)))
    return W


@pytest.mark.parametrize("levels,group,K", [(16, 64, 512), (8, 128, 1024), (4, 64, 768),
                                            (3, 16, 640), (16, 16, 256), (8, 32, 1536)])
def test_encode_properties(levels, group, K):
    rng = np.random.default_rng(levels * 7 + K)
    W = student_rows(rng, 24, K)
    e = enc.encode(W, levels, group, seed=11)
    G = e.u.reshape(24, K // group, group)
    np.testing.assert_allclose(np.mean(G * G, axis=-1), 1.0, rtol=1e-12)
    # the stored scale is the RMS of the rotated group rounded to fp16
    V = hd.rotate(W, 11).reshape(24, K // group, group)
    np.testing.assert_array_equal(e.scales, enc.fp16_bits(np.sqrt(np.mean(V * V, -1))))
    # snap equals brute-force nearest centroid away from thresholds
    c = cb.centroids(levels)
    nearest = np.argmin(np.abs(e.u[..., None] - c), axis=-1)
    far = ~enc.near_threshold(e.u, levels)
    np.testing.assert_array_equal(e.idx[far], nearest[far])
    # codes unpack to the indices
    np.testing.assert_array_equal(enc.unpack(e.codes, levels, K), e.idx)
    # per-element distortion close to that of Gaussian groups of the same size
    err = np.mean((e.u - c[e.idx]) ** 2)
    want = gaussian_group_distortion(levels, group, rng)
    assert abs(err - want) / want < 0.15


def gaussian_group_distortion(levels, group, rng, n=400_000):
    """MSE of the snap on i.i.d. Gaussian groups normalized by their own RMS, by sampling
    and brute-force nearest centroid (small groups have lighter tails than N(0,1))."""
    z = rng.standard_normal((n // group, group))
    u = z / np.sqrt(np.mean(z * z, axis=1, keepdims=True))
    c = cb.centroids(levels)
    nearest = np.argmin(np.abs(u[..., None] - c), axis=-1)
    return np.mean((u - c[nearest]) ** 2)


def test_distortion_statistical_large():
    # rotated heavy-tailed rows quantize like Gaussian groups
    rng = np.random.default_rng(99)
    W = student_rows(rng, 64, 4096)
    for levels, group in ((16, 64), (8, 128), (4, 64), (3, 16), (16, 16)):
        e = enc.encode(W, levels, group, seed=0)
        c = cb.centroids(levels)
        err = np.mean((e.u - c[e.idx]) ** 2)
        want = gaussian_group_distortion(levels, group, rng)
        assert abs(err - want) / want < 0.04, (levels, group, err, want)
        if group >= 64:  # large groups approach the N(0,1) codebook distortion
            assert abs(err - cb.distortion(levels)) / cb.distortion(levels) < 0.06


def test_power_of_two_scaling():
    rng = np.random.default_rng(3)
    W = student_rows(rng, 8, 512)
    a = enc.encode(W, 8, 64, seed=1)
    b = enc.encode(W * 4.0, 8, 64, seed=1)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(enc.fp16_value(b.scales), 4.0 * enc.fp16_value(a.scales))


def test_chunk_invariance():
    rng = np.random.default_rng(4)
    W = student_rows(rng, 40, 768)
    whole = enc.encode(W, 4, 32, seed=2)
    parts = [enc.encode(W[a:a + 7], 4, 32, seed=2) for a in range(0, 40, 7)]
    np.testing.assert_array_equal(np.concatenate([p.codes for p in parts]), whole.codes)
    np.testing.assert_array_equal(np.concatenate([p.scales for p in parts]), whole.scales)


def test_zero_rows():
    W = np.zeros((2, 256))
    W[1, :] = 1.0
    for levels in (3, 4, 8, 16):
        e = enc.encode(W, levels, 64, seed=0)
        assert np.all(e.scales[0] == 0)
        assert np.all(enc.dequant(e.codes[:1], e.scales[:1], levels, 64, 256) == 0.0)
        # u = 0 sits on the middle threshold of an even codebook (tie goes low); for the
        # ternary codebook it is the zero level
        want = levels // 2 - 1 if levels % 2 == 0 else 1
        assert np.all(e.idx[0] == want)


def test_constant_row_rotates_to_spike():
    # a constant row with all signs +1 would rotate to a single spike; the random signs
    # spread it: rotated values take +-1/sqrt(K) multiples, RMS equals the original RMS
    K = 1024
    W = np.ones((1, K))
    V = hd.rotate(W, 0)
    assert np.isclose(np.sqrt(np.mean(V * V)), 1.0)
    assert np.max(np.abs(V)) < 0.25 * np.sqrt(K)


def test_dequant_worked_examples():
    # Hand-built rows: known indices packed by the (separately pinned) packers, fp16 scales
    # with exact values, and the expected weights written out as centroid times the scale of
    # element j's group j // g. A wrong group mapping, index order or scale decode fails.
    c8 = cb.centroids(8)
    idx = np.array(list(range(8)) + list(range(7, -1, -1)) + list(range(8)) + list(range(7, -1, -1)))
    words = enc.pack(idx[None, :], 8)
    scales = np.array([[0x3800, 0x4200]], dtype=np.uint16)  # 0.5, 3.0
    got = enc.dequant(words, scales, 8, 16, 32)[0]
    want = np.array([c8[i] * (0.5 if j < 16 else 3.0) for j, i in enumerate(idx)])
    np.testing.assert_array_equal(got, want)
    # trits: K = 64 in four 16-element groups, digit j % 3 of element j
    c3 = cb.centroids(3)
    tidx = np.arange(64) % 3
    tw = enc.pack(tidx[None, :], 3)
    ts = np.array([[0x3E00, 0x3400, 0x4000, 0x3C00]], dtype=np.uint16)  # 1.5, 0.25, 2.0, 1.0
    got = enc.dequant(tw, ts, 3, 16, 64)[0]
    sv = [1.5, 0.25, 2.0, 1.0]
    want = np.array([c3[t] * sv[j // 16] for j, t in enumerate(tidx)])
    np.testing.assert_array_equal(got, want)
    assert c3[1] == 0.0 and c3[0] == -c3[2]


# Thresholds of the 3-level and 8-level codebooks written out from the closed form and the
# Max (1960) table rather than taken from the oracle: the ternary midpoint c/2 with c the
# root of c = phi(c/2) / (1 - Phi(c/2)), and the 3-bit midpoints of the pinned centroids.
HAND_THRESHOLDS = {3: [-0.6120, 0.6120], 8: [-1.7479, -1.0500, -0.5005, 0.0, 0.5005, 1.0500, 1.7479]}


@pytest.mark.parametrize("levels", [3, 8])
def test_near_threshold_band_edges(levels):
    # u placed 0.9e-6 and 1.1e-6 from each threshold (the band is 1e-6 wide in normalized
    # units); the hand values above locate the thresholds to 1e-4, then the exact fp64
    # threshold is the one the oracle uses, so the offsets are taken from it
    t = cb.thresholds(levels)
    assert np.allclose(t, HAND_THRESHOLDS[levels], atol=1.5e-4)
    inside = np.concatenate([t - 0.9e-6, t + 0.9e-6, t])
    outside = np.concatenate([t - 1.1e-6, t + 1.1e-6])
    assert np.all(enc.near_threshold(inside, levels, 1e-6))
    assert not np.any(enc.near_threshold(outside, levels, 1e-6))
    # far from every threshold, including the centroids themselves and large |u|
    far = np.concatenate([cb.centroids(levels), [-9.0, 9.0]])
    assert not np.any(enc.near_threshold(far, levels, 1e-6))
    # the mask keeps the input's shape
    assert enc.near_threshold(inside.reshape(-1, 1), levels).shape == (inside.size, 1)
