"""Pins of the oracle's bit and trit packing: hand-worked words and round trips."""

import numpy as np
import pytest

from oracle import encode as enc


def test_golden_words(golden):
    rows = golden("pack_words.txt")
    assert len(rows) >= 8
    for fmt, idx_s, words_s in rows:
        idx = np.array([[int(v) for v in idx_s.split(",")]])
        want = np.array([[int(w, 16) for w in words_s.split(",")]], dtype=np.uint32)
        if fmt == "t":
            got = enc.pack_trits(idx)
            back = enc.unpack_trits(got, idx.shape[1])
        else:
            b = int(fmt[1:])
            got = enc.pack_bits(idx, b)
            back = enc.unpack_bits(got, b, idx.shape[1])
        np.testing.assert_array_equal(got, want, err_msg=f"{fmt} {idx_s}")
        np.testing.assert_array_equal(back, idx)


def test_trit_word_fits():
    assert 3 ** 20 < 2 ** 32 <= 3 ** 21
    top = enc.pack_trits(np.full((1, 20), 2))
    assert int(top[0, 0]) == 3 ** 20 - 1


@pytest.mark.parametrize("levels,K", [(16, 512), (8, 4096), (4, 7168), (16, 2048), (3, 2048),
                                      (3, 768), (16, 4096), (16, 1536), (8, 33), (3, 21)])
def test_round_trip(levels, K):
    rng = np.random.default_rng(levels * 100000 + K)
    idx = rng.integers(0, levels, size=(3, K))
    words = enc.pack(idx, levels)
    assert words.dtype == np.uint32
    assert words.shape == (3, enc.words_per_row(K, levels))
    np.testing.assert_array_equal(enc.unpack(words, levels, K), idx)


def test_words_per_row():
    assert enc.words_per_row(4096, 8) == 384
    assert enc.words_per_row(7168, 4) == 448
    assert enc.words_per_row(2048, 16) == 256
    assert enc.words_per_row(2048, 3) == 103
    assert enc.words_per_row(768, 3) == 39
    assert enc.words_per_row(512, 16) == 64


def test_padding_bits_zero():
    idx = np.full((1, 11), 7)
    w = enc.pack_bits(idx, 3)
    assert int(w[0, 1]) == 1  # only stream bit 32 is set in the second word
    t = enc.pack_trits(np.full((1, 21), 2))
    assert int(t[0, 1]) == 2  # padding digits of the last word are 0


def test_eight_bit_words_are_bytes():
    # 8-bit codes (the 256-level KV-cache codebook): element j is byte j % 4 of word j // 4
    from oracle import encode as enc
    idx = np.array([[1, 2, 3, 4, 255, 0, 128, 7]])
    w = enc.pack(idx, 256)
    assert w.tolist() == [[0x04030201, 0x078000FF]]
    np.testing.assert_array_equal(enc.unpack(w, 256, 8), idx)
