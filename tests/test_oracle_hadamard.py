"""Pins of the oracle's Hadamard matrices, signs and rotation.

* Sylvester order 2^k equals scipy.linalg.hadamard and the closed form
  H[i, j] = (-1)^popcount(i & j).
* Paley matrices: entries +-1, H H^T = m I; the quadratic character agrees with Euler's
  criterion a^((q-1)/2) mod q; Paley I matrices are of skew type (H + H^T = 2I).
* SplitMix64: the first outputs for seed 0 equal the published ones
  (tests/golden/splitmix64_seed0.txt), and the counter form equals stepping the generator.
* Rotation: R e_j = s_j H[:, j] / sqrt(K) with H from the closed form (this fixes "signs
  first, then H" and the orientation), R R^T = I, the Kronecker (reshape) evaluation
  equals the dense matrix, the normalized Sylvester transform is an involution, and a
  heavy-tailed vector comes out close to Gaussian (excess kurtosis near 0).
"""

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard as hd


def stepped_signs(seed, n):
    """Signs from stepping the published SplitMix64 generator (state += gamma, then mix)."""
    state, out = seed, []
    for _ in range(n):
        state = (state + 0x9E3779B97F4A7C15) % 2 ** 64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) % 2 ** 64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) % 2 ** 64
        out.append(-1.0 if (z ^ (z >> 31)) >> 63 else 1.0)
    return np.array(out)


def popcount_sign(n):
    i = np.arange(n)
    bits = np.bitwise_and.outer(i, i)
    pc = np.array([bin(int(v)).count("1") for v in bits.ravel()]).reshape(n, n)
    return np.where(pc % 2 == 0, 1.0, -1.0)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 256, 1024])
def test_sylvester_matches_library_and_closed_form(n):
    H = hd.sylvester(n)
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(n))
    if n <= 256:
        np.testing.assert_array_equal(H, popcount_sign(n))


@pytest.mark.parametrize("q", [11, 13, 19])
def test_quadratic_character_euler(q):
    chi = hd.quadratic_character(q)
    for a in range(1, q):
        e = pow(a, (q - 1) // 2, q)
        assert chi[a] == (1 if e == 1 else -1)
    assert chi[0] == 0


@pytest.mark.parametrize("m", [12, 20, 28])
def test_paley_is_hadamard(m):
    H = hd.hadamard_m(m)
    assert H.shape == (m, m)
    assert set(np.unique(H)) == {-1.0, 1.0}
    np.testing.assert_array_equal(H @ H.T, m * np.eye(m))
    if m in (12, 20):
        np.testing.assert_array_equal(H + H.T, 2 * np.eye(m))  # skew type
        assert np.all(H[0] == 1.0) and np.all(H[1:, 0] == -1.0)


def test_paley2_structure():
    # blocks (i, j) are S_ij [[1,1],[1,-1]] for i != j and [[1,-1],[-1,-1]] on the diagonal
    H = hd.hadamard_m(28)
    for i in range(14):
        np.testing.assert_array_equal(H[2 * i:2 * i + 2, 2 * i:2 * i + 2], [[1, -1], [-1, -1]])
    np.testing.assert_array_equal(H[0:2, 2:4], [[1, 1], [1, -1]])  # S_01 = 1


@pytest.mark.parametrize("K", [16, 512, 768, 1536, 640, 2048])
def test_kronecker_hadamard_orthogonal(K):
    H = hd.hadamard(K)
    np.testing.assert_array_equal(H @ H.T, K * np.eye(K))


def test_split_dim():
    assert hd.split_dim(4096) == (1, 4096)
    assert hd.split_dim(7168) == (28, 256)
    assert hd.split_dim(1536) == (12, 128)
    assert hd.split_dim(768) == (12, 64)
    assert hd.split_dim(640) == (20, 32)
    for bad in (6, 100, 4864, 0):
        with pytest.raises(ValueError):
            hd.split_dim(bad)


def test_splitmix64_published(golden):
    want = [int(r[0], 16) for r in golden("splitmix64_seed0.txt")]
    assert hd.splitmix64_outputs(0, len(want)) == want


def test_splitmix64_counter_equals_stepping():
    state, seq = 12345, []
    for _ in range(50):
        state = (state + 0x9E3779B97F4A7C15) % 2 ** 64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) % 2 ** 64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) % 2 ** 64
        seq.append(z ^ (z >> 31))
    assert hd.splitmix64_outputs(12345, 50) == seq
    s = hd.signs(12345, 50)
    np.testing.assert_array_equal(s, [-1.0 if v >> 63 else 1.0 for v in seq])


def test_signs_balanced():
    s = hd.signs(0, 4096)
    assert set(np.unique(s)) == {-1.0, 1.0}
    assert abs(s.mean()) < 0.06


@pytest.mark.parametrize("K", [8, 64, 512])
def test_rotation_columns_closed_form(K):
    seed = 7
    s = stepped_signs(seed, K)
    Hc = popcount_sign(K)
    eye = np.eye(K)
    R_cols = hd.rotate(eye, seed)  # row j is R e_j
    np.testing.assert_allclose(R_cols, (Hc * s[None, :]).T / np.sqrt(K), atol=1e-15)


@pytest.mark.parametrize("K", [512, 768, 640, 1536])
def test_rotation_orthonormal_and_forms_agree(K):
    rng = np.random.default_rng(K)
    X = rng.standard_normal((5, K))
    A = hd.rotate(X, 3)
    B = hd.rotate_dense(X, 3)
    np.testing.assert_allclose(A, B, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(A, axis=1), np.linalg.norm(X, axis=1), rtol=1e-13)
    np.testing.assert_allclose(hd.unrotate(A, 3), X, atol=1e-12)
    R = hd.rotation_matrix(K, 3)
    np.testing.assert_allclose(R @ R.T, np.eye(K), atol=1e-13)


@pytest.mark.slow
def test_rotation_7168_forms_agree():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((2, 7168))
    np.testing.assert_allclose(hd.rotate(X, 0), hd.rotate_dense(X, 0), atol=1e-11)


def test_sylvester_involution():
    n = 1024
    H = hd.sylvester(n) / np.sqrt(n)
    np.testing.assert_allclose(H @ H, np.eye(n), atol=1e-13)


def test_rotation_gaussianizes():
    # heavy-tailed row with a few large outliers: excess kurtosis far above 0 before,
    # close to 0 (Gaussian) after the randomized rotation
    rng = np.random.default_rng(5)
    K = 4096
    x = rng.standard_t(3, K)
    x[rng.choice(K, 8, replace=False)] *= 50.0
    def excess_kurtosis(v):
        v = v - v.mean()
        return np.mean(v ** 4) / np.mean(v ** 2) ** 2 - 3.0
    assert excess_kurtosis(x) > 50
    assert abs(excess_kurtosis(hd.rotate(x, 0))) < 0.5
