"""Fixed Gaussian Lloyd-Max codebooks, computed in fp64 by Lloyd iteration.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: turboquant-mlx "How it works", section "Quantizing a weight, with no data" (third
bullet: each scaled weight snaps to the nearest centroid of the Lloyd-Max quantizer for a
Gaussian; one fixed codebook per bit width, a constant rather than something fitted) and
section "The ternary tier (1.58 bits)" (three levels {-c, 0, +c}; two levels {-c, +c} for
1 bit).

Lloyd's two optimality conditions for a scalar quantizer of the N(0,1) density:
  * every decision threshold is the midpoint of its two neighbouring centroids;
  * every centroid is the conditional mean of N(0,1) over its cell,
        E[X | a < X <= b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)).
Alternating the two from any ordered start converges to the unique fixed point (the
density is log-concave). Mean squared error at the fixed point is
        D = E[X^2] - sum_k P(cell k) c_k^2 = 1 - sum_k p_k c_k^2.

Reading taken here (the page gives no numbers): the iterate is kept exactly symmetric,
c_k = -c_{L-1-k}, by averaging each centroid with the negated mirror one after every
update. The fixed point is symmetric because N(0,1) is; the averaging only removes rounding
noise, so that the middle threshold of an even codebook is exactly 0.0 and the middle
centroid of the ternary codebook is exactly 0.0.

Index order is ascending: index 0 is the most negative centroid. For the ternary codebook
index 0/1/2 is -c/0/+c.
"""

import math
from functools import lru_cache

import numpy as np

_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def pdf(x):
    """N(0,1) density; 0 at +-inf."""
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def upper_tail(x):
    """Q(x) = P(X > x) for X ~ N(0,1), through erfc so that the upper tail keeps precision."""
    if x == math.inf:
        return 0.0
    if x == -math.inf:
        return 1.0
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def cell_probability(a, b):
    """P(a < X <= b), a < b, evaluated on the side of zero where it does not cancel."""
    if a >= 0.0:
        return upper_tail(a) - upper_tail(b)
    if b <= 0.0:
        return upper_tail(-b) - upper_tail(-a)
    return 1.0 - upper_tail(-a) - upper_tail(b)


def cell_mean(a, b):
    """E[X | a < X <= b] = (phi(a) - phi(b)) / P(a < X <= b)."""
    return (pdf(a) - pdf(b)) / cell_probability(a, b)


def midpoints(c):
    """Decision thresholds of an ascending codebook: midpoints of neighbouring centroids."""
    c = np.asarray(c, dtype=np.float64)
    return (c[:-1] + c[1:]) / 2.0


def lloyd_step(c):
    """One Lloyd update: thresholds at midpoints, then centroids at cell means."""
    t = midpoints(c)
    edges = [-math.inf] + [float(v) for v in t] + [math.inf]
    new = np.array([cell_mean(edges[k], edges[k + 1]) for k in range(len(c))])
    return (new - new[::-1]) / 2.0  # keep the exact symmetry of N(0,1)


@lru_cache(maxsize=None)
def _solve(levels, tol, max_iter):
    L = levels
    # any strictly increasing symmetric start works; spread evenly over [-2, 2]
    c = np.array([-2.0 + 4.0 * (k + 0.5) / L for k in range(L)])
    for it in range(1, max_iter + 1):
        new = lloyd_step(c)
        delta = float(np.max(np.abs(new - c)))
        c = new
        if delta < tol:
            break
    else:
        raise RuntimeError(f"Lloyd iteration for L={L} did not converge in {max_iter} steps")
    t = midpoints(c)
    edges = [-math.inf] + [float(v) for v in t] + [math.inf]
    p = np.array([cell_probability(edges[k], edges[k + 1]) for k in range(L)])
    D = 1.0 - float(np.sum(p * c * c))
    return c, t, D, it


def lloyd_max(levels, tol=1e-15, max_iter=200000):
    """Return (centroids, thresholds, distortion, iterations) of the L-level N(0,1) quantizer.

    ``centroids`` is ascending, length L; ``thresholds`` has length L-1.
    """
    if levels < 2:
        raise ValueError("a codebook needs at least two levels")
    c, t, D, it = _solve(int(levels), float(tol), int(max_iter))
    return c.copy(), t.copy(), D, it


def centroids(levels):
    return lloyd_max(levels)[0]


def thresholds(levels):
    return lloyd_max(levels)[1]


def distortion(levels):
    return lloyd_max(levels)[2]


def thresholds_f32(levels):
    """Thresholds rounded once to binary32; the snap decision is taken in binary32."""
    return thresholds(levels).astype(np.float32)


def snap(u, levels):
    """Index of the nearest centroid: idx = #{k : u > t_k}, decided in binary32.

    ``u`` is the group-normalized value in fp64. Both u and the thresholds are rounded once
    to binary32 before the comparison. An exact tie with a threshold goes to the lower
    index (the comparison is strict).
    """
    u32 = np.asarray(u, dtype=np.float64).astype(np.float32)
    t32 = thresholds_f32(levels)
    return np.sum(u32[..., None] > t32, axis=-1).astype(np.int64)


SUPPORTED_LEVELS = (3, 4, 8, 16)
BITS_OF_LEVELS = {4: 2, 8: 3, 16: 4}
