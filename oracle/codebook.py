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

The 256-level codebook is the one 8-bit KV-cache keys use ("How it works", "The KV cache":
the same rotation and codebook compress the cache, 8-bit keys and 3-bit values).
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


def lloyd_jacobian(c):
    """Tridiagonal Jacobian of lloyd_step at c: (sub, diag, super) of d(new c)/d(c).

    With a = t_{k-1}, b = t_k and m = E[X | a < X <= b], differentiating the cell mean
    (phi(a) - phi(b)) / P(a < X <= b) gives dm/db = phi(b) (b - m) / P and
    dm/da = phi(a) (m - a) / P; each threshold is the mean of its two neighbours, so
    d/dc_{k-1} = dm/da / 2, d/dc_k = (dm/da + dm/db) / 2, d/dc_{k+1} = dm/db / 2."""
    L = len(c)
    t = midpoints(c)
    edges = [-math.inf] + [float(v) for v in t] + [math.inf]
    sub, diag, sup = np.zeros(L), np.zeros(L), np.zeros(L)
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        P = cell_probability(a, b)
        m = cell_mean(a, b)
        da = 0.0 if math.isinf(a) else pdf(a) * (m - a) / P
        db = 0.0 if math.isinf(b) else pdf(b) * (b - m) / P
        sub[k], diag[k], sup[k] = da / 2.0, (da + db) / 2.0, db / 2.0
    return sub, diag, sup


def solve_tridiagonal(sub, diag, sup, rhs):
    """Thomas algorithm: x with sub[k] x[k-1] + diag[k] x[k] + sup[k] x[k+1] = rhs[k]."""
    n = len(diag)
    cp, dp = np.zeros(n), np.zeros(n)
    cp[0], dp[0] = sup[0] / diag[0], rhs[0] / diag[0]
    for k in range(1, n):
        den = diag[k] - sub[k] * cp[k - 1]
        cp[k] = sup[k] / den
        dp[k] = (rhs[k] - sub[k] * dp[k - 1]) / den
    x = np.zeros(n)
    x[-1] = dp[-1]
    for k in range(n - 2, -1, -1):
        x[k] = dp[k] - cp[k] * x[k + 1]
    return x


def _mp_lloyd_residual_and_jacobian(c):
    """lloyd_step(c) - c and its tridiagonal Jacobian, in mpmath's working precision (the
    same formulas as lloyd_step and lloyd_jacobian)."""
    import mpmath as mp
    L = len(c)
    t = [(c[k] + c[k + 1]) / 2 for k in range(L - 1)]
    edges = [None] + t + [None]
    pdf_ = lambda x: mp.exp(-x * x / 2) / mp.sqrt(2 * mp.pi)
    g, sub, diag, sup = [], [], [], []
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        pa = mp.mpf(0) if a is None else pdf_(a)
        pb = mp.mpf(0) if b is None else pdf_(b)
        Qa = mp.mpf(1) if a is None else mp.erfc(a / mp.sqrt(2)) / 2
        Qb = mp.mpf(0) if b is None else mp.erfc(b / mp.sqrt(2)) / 2
        P = Qa - Qb
        m = (pa - pb) / P
        da = mp.mpf(0) if a is None else pa * (m - a) / P
        db = mp.mpf(0) if b is None else pb * (b - m) / P
        g.append(m - c[k])
        sub.append(da / 2)
        diag.append((da + db) / 2 - 1)
        sup.append(db / 2)
    return g, sub, diag, sup


@lru_cache(maxsize=None)
def _solve_newton(levels, lloyd_steps):
    """The same fixed point for a large codebook. Plain Lloyd iteration contracts too slowly
    at 256 levels (about 0.99985 per step), and the fixed point is ill-conditioned for the
    map's rounding errors (they are amplified about 10^4 times), so: Lloyd steps from the
    same start, Newton's method on lloyd_step(c) - c = 0 in fp64 (Jacobian lloyd_jacobian -
    I), then Newton in 40-digit arithmetic (mpmath) to finish; the result is exact to far
    below the binary32 resolution the kernels use."""
    import mpmath as mp
    L = levels
    c = np.array([-2.0 + 4.0 * (k + 0.5) / L for k in range(L)])
    for _ in range(lloyd_steps):
        c = lloyd_step(c)
    for _ in range(40):
        g = lloyd_step(c) - c
        sub, diag, sup = lloyd_jacobian(c)
        delta = solve_tridiagonal(sub, diag - 1.0, sup, -g)
        c = c + delta
        c = (c - c[::-1]) / 2.0
        if float(np.max(np.abs(delta))) < 1e-9:
            break
    with mp.workdps(40):
        cm = [mp.mpf(float(v)) for v in c]
        for it in range(1, 21):
            g, sub, diag, sup = _mp_lloyd_residual_and_jacobian(cm)
            # Thomas algorithm in mpmath
            n = L
            cp, dp = [mp.mpf(0)] * n, [mp.mpf(0)] * n
            cp[0], dp[0] = sup[0] / diag[0], -g[0] / diag[0]
            for k in range(1, n):
                den = diag[k] - sub[k] * cp[k - 1]
                cp[k] = sup[k] / den
                dp[k] = (-g[k] - sub[k] * dp[k - 1]) / den
            d = [mp.mpf(0)] * n
            d[-1] = dp[-1]
            for k in range(n - 2, -1, -1):
                d[k] = dp[k] - cp[k] * d[k + 1]
            cm = [cm[k] + d[k] for k in range(n)]
            cm = [(cm[k] - cm[n - 1 - k]) / 2 for k in range(n)]
            if max(abs(x) for x in d) < mp.mpf(10) ** -30:
                break
        else:
            raise RuntimeError(f"Newton polish for L={L} did not converge")
        c = np.array([float(x) for x in cm])
    t = midpoints(c)  # as for every codebook: midpoints of the (fp64) centroids
    edges = [-math.inf] + [float(v) for v in t] + [math.inf]
    p = np.array([cell_probability(edges[k], edges[k + 1]) for k in range(L)])
    D = 1.0 - float(np.sum(p * c * c))
    return c, t, D, lloyd_steps + it


def lloyd_max(levels, tol=1e-15, max_iter=200000):
    """Return (centroids, thresholds, distortion, iterations) of the L-level N(0,1) quantizer.

    ``centroids`` is ascending, length L; ``thresholds`` has length L-1. Codebooks of up to
    16 levels come from plain Lloyd iteration; larger ones (the 256-level table of 8-bit KV
    keys) from Lloyd steps finished by Newton's method on the same fixed-point equations.
    """
    if levels < 2:
        raise ValueError("a codebook needs at least two levels")
    if levels > 16:
        c, t, D, it = _solve_newton(int(levels), 2000)
    else:
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
    if levels > 16:
        # the same count for the 255 thresholds of the 8-bit codebook, without a
        # [.., 255] comparison array: #{k : t_k < u} by binary search (side='left')
        return np.searchsorted(t32, u32, side="left").astype(np.int64)
    return np.sum(u32[..., None] > t32, axis=-1).astype(np.int64)


SUPPORTED_LEVELS = (3, 4, 8, 16, 256)
BITS_OF_LEVELS = {4: 2, 8: 3, 16: 4, 256: 8}
