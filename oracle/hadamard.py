"""Hadamard matrices, rotation signs and the randomized Hadamard rotation, in fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Sources
  * turboquant-mlx "How it works", "Quantizing a weight, with no data", first bullet: a
    Hadamard matrix with random +-1 signs is applied to every weight row; and "Running a
    quantized layer": the rotation is orthonormal, so the layer rotates its input with the
    same matrix instead of un-rotating the weights.
  * your-ssd-is-a-gpu, section on quantization ("create_hadamard_matrix"): the Sylvester
    doubling [[H, H], [H, -H]] from [[1]], divided by sqrt(dim) to make it orthogonal.

Readings (the pages leave these open)
  * R = H_K . diag(s) / sqrt(K): signs first, then the Hadamard matrix, natural
    (Sylvester) order. It acts on each weight row along the input dimension K, and the
    same R acts on the activation x, so that (R w) . (R x) = w . x.
  * K that is not a power of two: K = m * 2^k with m in {12, 20, 28} and
    H_K = H_m (x) H_{2^k} (Kronecker product, element index i = a * 2^k + b). The
    m-point matrices come from Paley's constructions with the conventions below. The
    pages do not say which order-m Hadamard matrix is meant; any one satisfies
    H H^T = m I, which is the only property the method relies on.
  * Signs: s_i = -1 when the top bit of SplitMix64 output number i (counting from 0) of
    the generator seeded with ``seed`` is set, else +1. Output number i is
    mix64(seed + (i + 1) * 0x9E3779B97F4A7C15 mod 2^64), with Stafford's "variant 13"
    finalizer mix64 as published with SplitMix64 (Steele, Lea and Flood, OOPSLA 2014;
    Vigna's splitmix64.c).

Paley conventions
  chi(a): quadratic character mod prime q (0 for a = 0, +1 for a non-zero square,
  -1 otherwise). Jacobsthal matrix Q[a][b] = chi(a - b), a, b in 0..q-1.
  Paley I (q = 3 mod 4, order q + 1):  H = I + [[0, 1^T], [-1, Q]].
  Paley II (q = 1 mod 4, order 2(q + 1)):  S = [[0, 1^T], [1, Q]];
      H = S (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]].
  H_12 = Paley I (q = 11), H_20 = Paley I (q = 19), H_28 = Paley II (q = 13).
"""

import numpy as np

SUPPORTED_M = (1, 12, 20, 28)

_GOLDEN_GAMMA = 0x9E3779B97F4A7C15
_MASK64 = (1 << 64) - 1


def sylvester(n):
    """Natural-order Sylvester Hadamard matrix of order n (a power of two), entries +-1."""
    if n < 1 or n & (n - 1):
        raise ValueError(f"Sylvester order must be a power of two, got {n}")
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def quadratic_character(q):
    """chi over Z_q for a prime q, as an int array of length q."""
    squares = {(x * x) % q for x in range(1, q)}
    chi = np.zeros(q, dtype=np.int64)
    for a in range(1, q):
        chi[a] = 1 if a in squares else -1
    return chi


def jacobsthal(q):
    chi = quadratic_character(q)
    return np.array([[chi[(a - b) % q] for b in range(q)] for a in range(q)], dtype=np.float64)


def paley1(q):
    """Paley construction I, q prime with q = 3 (mod 4): a Hadamard matrix of order q + 1."""
    if q % 4 != 3:
        raise ValueError("Paley I needs q = 3 mod 4")
    n = q + 1
    C = np.zeros((n, n))
    C[0, 1:] = 1.0
    C[1:, 0] = -1.0
    C[1:, 1:] = jacobsthal(q)
    return np.eye(n) + C


def paley2(q):
    """Paley construction II, q prime with q = 1 (mod 4): a Hadamard matrix of order 2(q + 1)."""
    if q % 4 != 1:
        raise ValueError("Paley II needs q = 1 mod 4")
    n = q + 1
    S = np.zeros((n, n))
    S[0, 1:] = 1.0
    S[1:, 0] = 1.0
    S[1:, 1:] = jacobsthal(q)
    A = np.array([[1.0, 1.0], [1.0, -1.0]])
    B = np.array([[1.0, -1.0], [-1.0, -1.0]])
    return np.kron(S, A) + np.kron(np.eye(n), B)


def hadamard_m(m):
    """The m-point factor: 1, or a Paley matrix of order 12, 20 or 28."""
    if m == 1:
        return np.array([[1.0]])
    if m == 12:
        return paley1(11)
    if m == 20:
        return paley1(19)
    if m == 28:
        return paley2(13)
    raise ValueError(f"unsupported Hadamard factor m={m}")


def split_dim(K):
    """K = m * 2^k with m in SUPPORTED_M; returns (m, 2^k). The decomposition is unique:
    12, 20 and 28 have different odd parts (3, 5, 7)."""
    for m in (1, 12, 20, 28):
        if K % m == 0:
            P = K // m
            if P >= 1 and P & (P - 1) == 0:
                return m, P
    raise ValueError(f"K={K} is not m * 2^k with m in {SUPPORTED_M}")


def hadamard(K):
    """H_K = H_m (x) H_{2^k}; entries +-1; H H^T = K I."""
    m, P = split_dim(K)
    return np.kron(hadamard_m(m), sylvester(P))


def splitmix64_outputs(seed, n):
    """The first n outputs of SplitMix64 seeded with ``seed``, as Python ints."""
    out = []
    for i in range(n):
        z = (seed + (i + 1) * _GOLDEN_GAMMA) & _MASK64
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK64
        out.append(z ^ (z >> 31))
    return out


def signs(seed, n):
    """Rotation signs s_0..s_{n-1} in {-1.0, +1.0}: -1 where the output's top bit is set."""
    return np.array([-1.0 if (z >> 63) else 1.0 for z in splitmix64_outputs(seed, n)])


def rotation_matrix(K, seed):
    """R = H_K diag(s) / sqrt(K), dense (fp64)."""
    return hadamard(K) * signs(seed, K)[None, :] / np.sqrt(K)


def rotate_dense(X, seed):
    """Rows of X (shape [..., K]) mapped to R x, through the dense matrix."""
    X = np.asarray(X, dtype=np.float64)
    K = X.shape[-1]
    return X @ rotation_matrix(K, seed).T


def rotate(X, seed):
    """Rows of X mapped to R x through the Kronecker identity
    (H_m (x) H_P) vec(V) = vec(H_m V H_P^T) on the row-major [m][P] view of each row."""
    X = np.asarray(X, dtype=np.float64)
    K = X.shape[-1]
    m, P = split_dim(K)
    V = (X * signs(seed, K)).reshape(-1, m, P)
    V = np.einsum("ij,rjb->rib", hadamard_m(m), V)
    V = V @ sylvester(P).T
    return (V / np.sqrt(K)).reshape(X.shape)


def unrotate(Y, seed):
    """Rows of Y mapped to R^T y (inverse rotation)."""
    Y = np.asarray(Y, dtype=np.float64)
    K = Y.shape[-1]
    return Y @ rotation_matrix(K, seed)
