"""The matrix-core trit decode's division-free constants, proved over their whole input
ranges on the CPU (no GPU).

trit_digits81 (rotation_lloyd_max_amd/csrc/mfma_decode.hpp) splits a trit word v < 3^20
(twenty base-3 digits, "The ternary tier (1.58 bits)"; the pages name the per-weight
division as what made ternary slow, "Running a quantized layer") into five base-81 digits
with multiplies only:
    hi = umulhi(v, M1) >> S1          v / 6561 for every 32-bit v
    q1 = umul24(lo, M2) >> S2         lo / 81 for lo < 6561
    q4 = (hi * M3) >> 32              hi / 6561 for hi < 3^12
The constants are read from the kernel source, so the test checks what the GPU runs.
"""

import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "rotation_lloyd_max_amd", "csrc", "mfma_decode.hpp")


def constants():
    text = open(SRC).read()
    body = text[text.index("void trit_digits81"):]
    body = body[:body.index("\n}\n")]
    m1, s1 = map(int, re.search(r"__umulhi\(v, (\d+)u\) >> (\d+)", body).groups())
    m2, s2 = map(int, re.search(r"__umul24\(lo, (\d+)u\) >> (\d+)", body).groups())
    m2b, s2b = map(int, re.search(r"__umul24\(r, (\d+)u\) >> (\d+)", body).groups())
    m3 = int(re.search(r"\* (\d+)ull\) >> 32", body).group(1))
    assert (m2, s2) == (m2b, s2b)
    return m1, s1, m2, s2, m3


def divide_hi(v, m1, s1):
    v = np.asarray(v, dtype=np.uint64)
    return ((v * np.uint64(m1)) >> np.uint64(32)) >> np.uint64(s1)


def test_umulhi_divides_every_32_bit_word_by_6561():
    m1, s1, _, _, _ = constants()
    d, n = 6561, 32 + s1
    # round-up magic number: M d >= 2^n, and the excess M d - 2^n <= 2^s1 makes the
    # overshoot v e / (d 2^n) < 1/d for v < 2^32 (Granlund and Montgomery 1994, Thm 4.2)
    assert m1 * d >= 1 << n and m1 * d - (1 << n) <= 1 << s1
    # the overshoot grows with v and the residue d - 1 leaves the least room, so checking
    # every v = k d + d - 1 below 2^32, plus the last partial block, checks every v
    v = np.arange(d - 1, 1 << 32, d, dtype=np.uint64)
    np.testing.assert_array_equal(divide_hi(v, m1, s1), v // np.uint64(d))
    tail = np.arange(((1 << 32) // d) * d, 1 << 32, dtype=np.uint64)
    np.testing.assert_array_equal(divide_hi(tail, m1, s1), tail // np.uint64(d))
    low = np.arange(0, 1 << 20, dtype=np.uint64)
    np.testing.assert_array_equal(divide_hi(low, m1, s1), low // np.uint64(d))


def test_24_bit_multiplies_over_their_ranges():
    _, _, m2, s2, m3 = constants()
    lo = np.arange(6561, dtype=np.uint64)               # the remainder of v / 6561
    assert m2 < 1 << 24 and int(lo[-1]) < 1 << 24        # both operands fit v_mul_u32_u24
    np.testing.assert_array_equal((lo * np.uint64(m2)) >> np.uint64(s2), lo // np.uint64(81))
    hi = np.arange(3 ** 12, dtype=np.uint64)            # v / 6561 for v < 3^20
    assert m3 < 1 << 24 and int(hi[-1]) < 1 << 24
    np.testing.assert_array_equal((hi * np.uint64(m3)) >> np.uint64(32), hi // np.uint64(6561))


def digits81(v, c):
    """trit_digits81 written out in numpy with the source's constants."""
    m1, s1, m2, s2, m3 = c
    v = np.asarray(v, dtype=np.uint64)
    hi = divide_hi(v, m1, s1)
    lo = v - hi * np.uint64(6561)
    q1 = (lo * np.uint64(m2)) >> np.uint64(s2)
    q4 = (hi * np.uint64(m3)) >> np.uint64(32)
    r = hi - q4 * np.uint64(6561)
    q3 = (r * np.uint64(m2)) >> np.uint64(s2)
    return [lo - q1 * np.uint64(81), q1, r - q3 * np.uint64(81), q3, q4]


def test_five_digits_are_the_base_81_digits_of_every_word():
    c = constants()
    g = np.random.Generator(np.random.PCG64(7))
    top = 3 ** 20
    v = np.concatenate([np.arange(0, 1 << 18), np.arange(top - (1 << 18), top),
                        g.integers(0, top, 1 << 20)]).astype(np.uint64)
    q = digits81(v, c)
    w = v.copy()
    for k in range(5):
        np.testing.assert_array_equal(q[k], w % np.uint64(81))
        w //= np.uint64(81)
    # digit k of a word holds trits 4k .. 4k + 3 (least significant first)
    t = np.array([2, 0, 1, 1, 2, 2, 0, 0, 1, 0, 2, 1, 0, 0, 0, 2, 1, 2, 0, 1], dtype=np.uint64)
    word = int(np.sum(t * np.uint64(3) ** np.arange(20, dtype=np.uint64)))
    d = [int(x[0]) for x in digits81([word], c)]
    assert d == [int(t[4 * k] + 3 * t[4 * k + 1] + 9 * t[4 * k + 2] + 27 * t[4 * k + 3])
                 for k in range(5)]
