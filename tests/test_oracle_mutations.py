"""Planted mistakes in the oracle (on the CPU) must each fail a pin.

Each case monkeypatches one oracle function with a plausible mistake (a dropped sign
vector, a transposed operand, a wrong bit order, a wrong divisor, a threshold off the
midpoint) and checks that the corresponding pin, re-run against the mutated oracle,
fails. This shows the pins are sharp enough to notice such mistakes.
"""

import numpy as np
import pytest

from oracle import codebook as cb
from oracle import encode as enc
from oracle import hadamard as hd

from test_oracle_hadamard import popcount_sign, stepped_signs
from conftest import golden_lines


def rotation_pin(K=64, seed=7):
    s = stepped_signs(seed, K)
    want = (popcount_sign(K) * s[None, :]).T / np.sqrt(K)
    return np.allclose(hd.rotate(np.eye(K), seed), want, atol=1e-15)


def pack_pin():
    for fmt, idx_s, words_s in golden_lines("pack_words.txt"):
        idx = np.array([[int(v) for v in idx_s.split(",")]])
        want = np.array([[int(w, 16) for w in words_s.split(",")]], dtype=np.uint32)
        got = enc.pack_trits(idx) if fmt == "t" else enc.pack_bits(idx, int(fmt[1:]))
        if got.shape != want.shape or not np.array_equal(got, want):
            return False
    return True


def unit_rms_pin():
    rng = np.random.default_rng(0)
    e = enc.encode(rng.standard_t(4, (8, 256)), 8, 64, 0)
    return np.allclose(np.mean(e.u.reshape(8, 4, 64) ** 2, -1), 1.0, rtol=1e-12)


def stationarity_pin(L=8):
    from scipy import integrate, stats
    c, t, _, _ = cb.lloyd_max(L)
    edges = [-np.inf] + list(t) + [np.inf]
    for k in range(L):
        a, b = edges[k], edges[k + 1]
        m = integrate.quad(stats.norm.pdf, a, b)[0]
        f = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b)[0]
        if abs(f / m - c[k]) > 1e-9:
            return False
    return True


def test_pins_hold_unmutated():
    assert rotation_pin() and pack_pin() and unit_rms_pin() and stationarity_pin()


def test_dropped_signs_caught(monkeypatch):
    monkeypatch.setattr(hd, "signs", lambda seed, n: np.ones(n))
    assert not rotation_pin()


def test_transposed_rotation_caught(monkeypatch):
    def rotate_t(X, seed):
        X = np.asarray(X, dtype=np.float64)
        return X @ hd.rotation_matrix(X.shape[-1], seed)  # R^T instead of R
    monkeypatch.setattr(hd, "rotate", rotate_t)
    assert not rotation_pin()


def test_msb_first_bits_caught(monkeypatch):
    real = enc.pack_bits
    def msb_first(idx, b):
        rev = np.zeros_like(np.asarray(idx))
        for q in range(b):
            rev |= ((np.asarray(idx) >> q) & 1) << (b - 1 - q)
        return real(rev, b)
    monkeypatch.setattr(enc, "pack_bits", msb_first)
    assert not pack_pin()


def test_trit_digit_order_caught(monkeypatch):
    real = enc.pack_trits
    monkeypatch.setattr(enc, "pack_trits", lambda idx: real(np.asarray(idx)[:, ::-1]))
    assert not pack_pin()


def test_divide_by_rounded_scale_caught(monkeypatch):
    def encode_rounded(W, levels, group, seed):
        W = np.asarray(W, dtype=np.float64)
        rows, K = W.shape
        V = hd.rotate(W, seed).reshape(rows, K // group, group)
        r = enc.fp16_value(enc.fp16_bits(np.sqrt(np.mean(V * V, -1))))
        U = (V / r[..., None]).reshape(rows, K)
        idx = cb.snap(U, levels)
        return enc.Encoded(enc.pack(idx, levels), enc.fp16_bits(r), U, idx, r)
    monkeypatch.setattr(enc, "encode", encode_rounded)
    assert not unit_rms_pin()


def test_threshold_off_midpoint_caught(monkeypatch):
    cb._solve.cache_clear()
    monkeypatch.setattr(cb, "midpoints", lambda c: np.asarray(c)[:-1] * 0.75 + np.asarray(c)[1:] * 0.25)
    try:
        assert not stationarity_pin()
    finally:
        monkeypatch.undo()
        cb._solve.cache_clear()
