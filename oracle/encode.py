"""Encode (rotate -> group RMS -> fp16 scale -> snap -> pack), unpack and dequantize, fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: turboquant-mlx "How it works", section "Quantizing a weight, with no data"
(bullets: randomized Hadamard rotation; groups along the input dimension of 16/32/64/128
each divided by its root-mean-square; snap to the nearest Lloyd-Max centroid; indices
bit-packed into 32-bit words, 2, 3 or 4 bits each, with per-group scales stored alongside),
and section "The ternary tier (1.58 bits)" (twenty base-3 digits per 32-bit word; a
codebook of 2^b entries means bit-packed, one of 3 entries means trit-packed).

Readings (the pages leave these open)
  * Layout: codes [rows][words_per_row] uint32, scales [rows][K / group] as fp16 bit
    patterns, both row-major; rows are packed independently.
  * Bit packing: element j of a row occupies bits [b*j, b*j + b) of the row's
    little-endian bitstream, where bit p of the stream is bit (p mod 32) of word p // 32.
    A code may straddle two words (3 bits). words_per_row = ceil(K * b / 32); unused
    high bits of the last word are zero.
  * Trit packing: word w of a row holds elements 20w .. 20w + 19 as sum_k t_k 3^k with
    element 20w + k in digit k (least significant first); words_per_row = ceil(K / 20);
    padding digits are 0.
  * The stored scale is the group RMS r rounded once to fp16 (round to nearest even,
    saturating at 65504). Values are divided by the unrounded r; r = 0 gives u = 0.
  * The snap decision idx = #{k : u > t_k} is taken in binary32 (u and t each rounded
    once to binary32), ties to the lower index.
"""

from dataclasses import dataclass

import numpy as np

from . import codebook as cb
from . import hadamard as hd

FP16_MAX = 65504.0


def fp16_bits(r):
    """fp64 -> fp16 bit patterns, round to nearest even, saturating at the largest finite."""
    r = np.minimum(np.asarray(r, dtype=np.float64), FP16_MAX)
    return r.astype(np.float16).view(np.uint16)


def fp16_value(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bits_per_code(levels):
    if levels == 3:
        return None  # trit packed
    return cb.BITS_OF_LEVELS[levels]


def words_per_row(K, levels):
    if levels == 3:
        return -(-K // 20)
    return -(-K * bits_per_code(levels) // 32)


def pack_bits(idx, b):
    """idx [rows][K] ints in [0, 2^b) -> uint32 [rows][ceil(K*b/32)], LSB-first bitstream."""
    idx = np.asarray(idx, dtype=np.uint64)
    rows, K = idx.shape
    wpr = -(-K * b // 32)
    words = np.zeros((rows, wpr), dtype=np.uint64)
    j = np.arange(K)
    for q in range(b):  # bit q of code j goes to stream position b*j + q
        p = b * j + q
        bit = (idx >> np.uint64(q)) & np.uint64(1)
        # each stream position is written by exactly one (j, q), so adding is OR
        np.add.at(words, (slice(None), p // 32), bit << (p % 32).astype(np.uint64))
    return words.astype(np.uint32)


def unpack_bits(words, b, K):
    words = np.asarray(words, dtype=np.uint64)
    rows = words.shape[0]
    idx = np.zeros((rows, K), dtype=np.int64)
    j = np.arange(K)
    for q in range(b):
        p = b * j + q
        bit = (words[:, p // 32] >> (p % 32).astype(np.uint64)) & np.uint64(1)
        idx |= bit.astype(np.int64) << q
    return idx


_POW3 = np.array([3 ** k for k in range(20)], dtype=np.int64)


def pack_trits(idx):
    """idx [rows][K] ints in {0,1,2} -> uint32 [rows][ceil(K/20)], 20 base-3 digits per word."""
    idx = np.asarray(idx, dtype=np.int64)
    rows, K = idx.shape
    wpr = -(-K // 20)
    padded = np.zeros((rows, wpr * 20), dtype=np.int64)
    padded[:, :K] = idx
    return (padded.reshape(rows, wpr, 20) @ _POW3).astype(np.uint32)


def unpack_trits(words, K):
    w = np.asarray(words, dtype=np.int64).copy()
    rows, wpr = w.shape
    digits = np.zeros((rows, wpr, 20), dtype=np.int64)
    for k in range(20):
        digits[:, :, k] = w % 3
        w //= 3
    return digits.reshape(rows, wpr * 20)[:, :K]


def pack(idx, levels):
    if levels == 3:
        return pack_trits(idx)
    return pack_bits(idx, bits_per_code(levels))


def unpack(words, levels, K):
    if levels == 3:
        return unpack_trits(words, K)
    return unpack_bits(words, bits_per_code(levels), K)


@dataclass
class Encoded:
    codes: np.ndarray   # uint32 [rows][words_per_row]
    scales: np.ndarray  # uint16 fp16 bits [rows][K / group]
    u: np.ndarray       # fp64 [rows][K] group-normalized rotated values
    idx: np.ndarray     # int64 [rows][K] codebook indices
    r: np.ndarray       # fp64 [rows][K / group] unrounded group RMS


def encode(W, levels, group, seed):
    """Quantize the rows of W (shape [rows][K], any float dtype, read exactly as fp64)."""
    W = np.asarray(W, dtype=np.float64)
    if W.ndim != 2:
        raise ValueError("W must be 2-D [rows][K]")
    return encode_rotated(hd.rotate(W, seed), levels, group)      # v = R w


def encode_dense(W, R, levels, group):
    """The same quantizer with a dense orthogonal rotation R (shape [K][K]) in place of the
    randomized Hadamard one: v = R w for every row (VeloxQuant-MLX, "What already existed"
    and "Where the time actually went": a QR-derived rotation for input dimensions the fast
    Hadamard transform does not cover, such as 4864)."""
    W = np.asarray(W, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    return encode_rotated(W @ R.T, levels, group)


def encode_rotated(V, levels, group):
    """Group RMS -> fp16 scale -> snap -> pack of rows that are already rotated."""
    V = np.asarray(V, dtype=np.float64)
    if V.ndim != 2:
        raise ValueError("V must be 2-D [rows][K]")
    rows, K = V.shape
    if levels not in cb.SUPPORTED_LEVELS:
        raise ValueError(f"unsupported number of levels {levels}")
    if group not in (16, 32, 64, 128) or K % group:
        raise ValueError(f"group {group} must be 16/32/64/128 and divide K={K}")
    G = V.reshape(rows, K // group, group)
    r = np.sqrt(np.mean(G * G, axis=-1))                    # group RMS
    safe = np.where(r > 0.0, r, 1.0)
    U = np.where(r[..., None] > 0.0, G / safe[..., None], 0.0).reshape(rows, K)
    idx = cb.snap(U, levels)
    return Encoded(pack(idx, levels), fp16_bits(r), U, idx, r)


def near_threshold(u, levels, eps=1e-6):
    """Mask of values within eps of a decision threshold (fp64 distance)."""
    t = cb.thresholds(levels)
    return np.min(np.abs(np.asarray(u)[..., None] - t), axis=-1) <= eps


def dequant(codes, scales, levels, group, K):
    """w'_hat[i, j] = c[idx[i, j]] * scale[i, j // group] in the rotated basis (fp64)."""
    idx = unpack(codes, levels, K)
    c = cb.centroids(levels)
    s = fp16_value(scales)
    return c[idx] * np.repeat(s, group, axis=-1)


def dequant_unrotated(codes, scales, levels, group, K, seed):
    """w_hat = R^T w'_hat: the quantized weight in the original basis."""
    return hd.unrotate(dequant(codes, scales, levels, group, K), seed)


def kv_fetch(codes, scales, levels, group, K, seed):
    """The fetch half of a compressed KV cache: each stored row dequantized and rotated back
    ("your SSD is a GPU", KV-cache section: rotate, quantize, store, then dequantize and
    de-rotate; turboquant-mlx "How it works", "The KV cache": the weights' rotation and
    codebook, 8-bit keys and 3-bit values). Rows are (token, head) vectors of head_dim K."""
    return dequant_unrotated(codes, scales, levels, group, K, seed)
