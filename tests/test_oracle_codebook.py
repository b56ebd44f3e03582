"""Pins of the oracle's Lloyd-Max codebooks against facts that do not use its own formulas.

* 2 levels: closed form c = sqrt(2/pi), D = 1 - 2/pi.
* 4/8/16 levels: Max (1960) Table I values (tests/golden/lloyd_max_gaussian.txt): each
  oracle value lies within one unit of the table's last printed digit.
* Every level count: centroids are conditional means and D is the MSE, both by adaptive
  quadrature of the N(0,1) density (scipy.integrate.quad, scipy.stats.norm), i.e. not
  through the erf-based cell formulas the oracle iterates with.
* 3 levels: the one-parameter fixed point c = phi(c/2) / (1 - Phi(c/2)) by root finding.
* Monte Carlo: nearest-centroid quantization of N(0,1) samples by brute force argmin has
  the oracle's distortion and agrees with the threshold snap.
* 256 levels (8-bit KV-cache keys): the same quadrature stationarity and MSE, the
  Panter-Dite high-resolution distortion (sqrt(3) pi / 2) 4^-b within 1 %, a fixed point of
  the plain Lloyd map, Monte Carlo distortion and snap.
"""

import math

import numpy as np
import pytest
from scipy import integrate, optimize, stats

from oracle import codebook as cb

LEVELS = (2, 3, 4, 8, 16, 256)


def test_two_levels_closed_form():
    c, t, D, _ = cb.lloyd_max(2)
    assert abs(c[1] - math.sqrt(2 / math.pi)) < 1e-14
    assert c[0] == -c[1]
    assert t[0] == 0.0
    assert abs(D - (1 - 2 / math.pi)) < 1e-14


def test_max_1960_table(golden):
    rows = golden("lloyd_max_gaussian.txt")
    assert rows
    for row in rows:
        L, kind, texts = int(row[0]), row[1], row[2:]
        vals = [float(v) for v in texts]
        # one unit in the last printed digit: the table's rounding plus its known
        # last-digit slips (it was computed in 1960)
        half_ulp = [10.0 ** -(len(v.split(".")[1]) if "." in v else 0) + 1e-12
                    for v in texts]
        c, t, D, _ = cb.lloyd_max(L)
        if kind == "centroids":
            got = c[L // 2:]
        elif kind == "thresholds":
            got = t[(L - 1) // 2:]
        elif kind == "distortion":
            # rounding of the printed digits, or 1e-5 for Max's 16-level entry 0.009497,
            # which is 4e-6 below the fixed point 0.0095010
            assert abs(D - vals[0]) <= max(half_ulp[0], 1e-5), (L, D)
            continue
        else:
            raise AssertionError(kind)
        assert len(got) == len(vals)
        for g, v, h in zip(got, vals, half_ulp):
            assert abs(g - v) <= h, (L, kind, g, v)


@pytest.mark.parametrize("L", LEVELS)
def test_stationarity_by_quadrature(L):
    c, t, D, _ = cb.lloyd_max(L)
    edges = [-np.inf] + list(t) + [np.inf]
    phi = stats.norm.pdf
    mse = 0.0
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        mass = integrate.quad(phi, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        first = integrate.quad(lambda x: x * phi(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(first / mass - c[k]) < 1e-9, (L, k)
        mse += integrate.quad(lambda x: (x - c[k]) ** 2 * phi(x), a, b,
                              epsabs=1e-14, epsrel=1e-13)[0]
    assert abs(mse - D) < 1e-10
    # thresholds are midpoints and the codebook is symmetric and increasing
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])
    np.testing.assert_allclose(t, (c[:-1] + c[1:]) / 2, rtol=0, atol=0)


def test_ternary_fixed_point():
    def f(c):
        return c - stats.norm.pdf(c / 2) / stats.norm.sf(c / 2)
    root = optimize.brentq(f, 0.5, 2.5, xtol=1e-15)
    c, t, D, _ = cb.lloyd_max(3)
    assert c[1] == 0.0
    assert abs(c[2] - root) < 1e-12
    assert abs(t[1] - root / 2) < 1e-12
    assert abs(c[2] - 1.224) < 1e-3 and abs(t[1] - 0.612) < 1e-3


def test_middle_threshold_is_exact_zero():
    for L in (2, 4, 8, 16, 256):
        assert cb.thresholds(L)[L // 2 - 1] == 0.0


@pytest.mark.parametrize("L", (3, 4, 8, 16, 256))
def test_monte_carlo_nearest_centroid(L):
    rng = np.random.default_rng(1234 + L)
    x = rng.standard_normal(1_000_000 if L <= 16 else 200_000)
    c = cb.centroids(L)
    nearest = np.argmin(np.abs(x[:, None] - c[None, :]), axis=1)
    mse = np.mean((x - c[nearest]) ** 2)
    D = cb.distortion(L)
    # std of the MSE estimate is below 0.2% of D at these sizes for up to 16 levels; at
    # 256 levels one sample beyond the outermost centroid (|x| > 4.6) moves the estimate
    # by about 1 %, so the bound is wider there (quadrature pins D itself)
    assert abs(mse - D) / D < (0.01 if L <= 16 else 0.05)
    idx = cb.snap(x, L)
    far = ~np.any(np.abs(x[:, None] - cb.thresholds(L)[None, :]) < 1e-6, axis=1)
    np.testing.assert_array_equal(idx[far], nearest[far])


def test_snap_tie_goes_low():
    for L in (4, 8, 16):
        t = cb.thresholds(L)
        # a value exactly on a (binary32) threshold goes to the lower cell
        u = np.array([float(np.float32(v)) for v in t])
        np.testing.assert_array_equal(cb.snap(u, L), np.arange(L - 1))


def test_256_levels_panter_dite_and_lloyd_fixed_point():
    # high-resolution theory: D ~ (sqrt(3) pi / 2) 4^-b for a Gaussian quantized with 2^b
    # optimal levels; at b = 8 the asymptote is within 1 % of the exact optimum
    c, t, D, _ = cb.lloyd_max(256)
    pd = math.sqrt(3.0) * math.pi / 2.0 * 4.0 ** -8
    assert abs(D / pd - 1.0) < 0.01
    assert 4.0e-5 < D < 4.2e-5
    # the result is a fixed point of the plain Lloyd map itself (to its rounding)
    assert np.max(np.abs(cb.lloyd_step(c) - c)) < 1e-13
    # and it sits between the 16-level table's neighbours: 8-bit refines 4-bit
    assert D < cb.distortion(16) / 200
    # tails: the outermost centroid is the conditional mean beyond the last threshold
    tail = stats.norm.pdf(t[-1]) / stats.norm.sf(t[-1])
    assert abs(c[-1] - tail) < 1e-12


def test_256_level_snap_counts_thresholds():
    # the searchsorted count used for 255 thresholds equals the comparison count
    rng = np.random.default_rng(99)
    u = np.concatenate([rng.standard_normal(20000) * 1.5, cb.thresholds(256)[::7]])
    t32 = cb.thresholds_f32(256)
    want = np.sum(u.astype(np.float32)[:, None] > t32[None, :], axis=1)
    np.testing.assert_array_equal(cb.snap(u, 256), want)
