"""Parity helpers: compare the HIP path's results with the oracle's, on the same bytes.

Rules
  codes    bit-exact, except at elements whose oracle-normalized value u lies within 1e-6
           of a decision threshold; those are counted and may be at most 1e-6 of the
           elements (so a small layer must match exactly).
  scales   bit-exact, except where the oracle's group RMS lies within 1e-6 (relative) of
           an fp16 rounding boundary.
  outputs  |y_gpu - y_oracle| <= 2e-3 * ||x|| * ||w'_hat_row|| for every row, with the
           oracle evaluated in fp64 on the GPU's own codes and scales (isolating decode
           and multiply) and on its own codes (end to end).

A second, sharper output bound is checked beside the required one. The kernels hold the
rotated input x' in fp16 (scaled by a power of two), the centroids in fp16 and, in the
matrix-core kernels, each decoded weight c * scale rounded to fp16, and they accumulate in
fp32. Each of those roundings moves a product w_j x'_j by at most 2^-11 of itself, and a
chain of d fp32 additions moves the sum by at most d 2^-24 of the sum of |terms|, so
    |y_gpu - y_oracle| <= (3 2^-11 + d 2^-24) sum_j |w'_hat_j x'_j| + (rotation error),
with d = K/16 + 64 and the fp32 rotation error (at most log2(K) 2^-24 ||x|| per entry of
x', and 2^-17 of the H_64 X product on the matrix-core rotation) taken as
2^-16 ||w'_hat||_1 ||x||_2.

The sharpest check feeds pre-rotated inputs of +-1 (exact in every input dtype and in the
kernels' scaled fp16): then the only roundings left are the fp16 centroids (and, in the
matrix-core kernels, the fp16 products c * scale), which `kernel_weights` reproduces
exactly, and the fp32 sums, so |y_gpu - x' . w16| <= d 2^-24 sum_j |w16_j x'_j|. One wrong
code anywhere in a row of up to 6144 4-bit codes moves y by more than that
(tests/test_oracle_sharp.py plants such flips).
"""

import numpy as np

from oracle import codebook as ocb
from oracle import encode as oenc
from oracle import ops as oops


def torch_to_np(t):
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def as_f64(t):
    """Exact fp64 value of a torch tensor's elements (float32 / bfloat16 / float16)."""
    import torch
    a = t.detach().cpu()
    if a.dtype == torch.bfloat16:
        return (a.view(torch.int16).numpy().view(np.uint16).astype(np.uint32) << 16).view(
            np.float32).astype(np.float64)
    return a.to(torch.float64).numpy() if a.dtype != torch.float64 else a.numpy()


def check_codes(gpu_codes, ref, levels, K, tag=""):
    """gpu_codes uint32 [rows][wpr]; ref an oracle Encoded. Returns the mismatch count."""
    gpu_codes = np.asarray(gpu_codes, dtype=np.uint32).reshape(ref.codes.shape)
    gidx = oenc.unpack(gpu_codes, levels, K)
    mism = gidx != ref.idx
    n = int(mism.sum())
    if n:
        near = oenc.near_threshold(ref.u, levels, 1e-6)
        bad = mism & ~near
        assert not bad.any(), f"{tag}: {int(bad.sum())} code mismatches away from thresholds"
        assert n <= 1e-6 * mism.size, f"{tag}: {n} near-threshold mismatches of {mism.size}"
        ok_rows = ~mism.any(axis=1)
        np.testing.assert_array_equal(gpu_codes[ok_rows], ref.codes[ok_rows])
    else:
        np.testing.assert_array_equal(gpu_codes, ref.codes, err_msg=tag)
    return n


def check_scales(gpu_scales, ref, tag=""):
    gpu_scales = np.asarray(gpu_scales, dtype=np.uint16).reshape(ref.scales.shape)
    mism = gpu_scales != ref.scales
    if mism.any():
        lo = oenc.fp16_bits(ref.r * (1 - 1e-6))
        hi = oenc.fp16_bits(ref.r * (1 + 1e-6))
        ambiguous = lo != hi
        assert not (mism & ~ambiguous).any(), f"{tag}: scale mismatches away from fp16 ties"
    return int(mism.sum())


def check_outputs(y_gpu, y_ref, bound, tag=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    assert np.all(np.isfinite(y_gpu)), f"{tag}: non-finite outputs"
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert np.all(err <= bound), f"{tag}: max err/bound = {worst:.3g}"
    return worst


def qmv_reference(codes, scales, levels, group, K, seed, x):
    """(y, bound) from the oracle for one dense weight and input(s) x."""
    y = oops.qmv(codes, scales, levels, group, K, seed, x)
    b = oops.row_bound(codes, scales, levels, group, K, x)
    return y, b


def acc_depth(K):
    """Longest chain of fp32 additions allowed for a row of length K."""
    return K // 16 + 64


def apriori_bound(codes, scales, levels, group, K, seed, x):
    """The a-priori rounding bound of the module docstring, per (input, row)."""
    Wq = oenc.dequant(codes, scales, levels, group, K)
    x = np.asarray(x, dtype=np.float64)
    xr = ohd_rotate(x, seed)
    terms = np.abs(xr) @ np.abs(Wq).T
    rel = 3.0 * 2.0 ** -11 + acc_depth(K) * 2.0 ** -24
    xn = np.linalg.norm(x, axis=-1)
    return rel * terms + 2.0 ** -16 * np.multiply.outer(xn, np.sum(np.abs(Wq), axis=-1))


def ohd_rotate(x, seed):
    from oracle import hadamard as ohd
    return ohd.rotate(x, seed)


def qmv_reference(codes, scales, levels, group, K, seed, x):
    """(y, bound) from the oracle for one dense weight and input(s) x; the bound is the
    smaller of the required 2e-3 ||x|| ||w'_hat_i|| and the a-priori rounding bound."""
    y = oops.qmv(codes, scales, levels, group, K, seed, x)
    b = oops.row_bound(codes, scales, levels, group, K, x)
    a = apriori_bound(codes, scales, levels, group, K, seed, x)
    return y, np.minimum(b, a)


def fp16(a):
    """fp64 -> the nearest fp16 value (ties to even), returned as fp64."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def kernel_weights(codes, scales, levels, group, K, rounded_products):
    """The decoded weights [rows][K] as the kernels multiply them: the centroid rounded to
    fp16 times the fp16 group scale (exact; the qmv kernel scales each group's fp32 partial
    sum), and with rounded_products that product rounded to fp16 (the matrix-core kernels
    form c * scale with one fp16 multiply)."""
    idx = oenc.unpack(codes, levels, K)
    c16 = fp16(ocb.centroids(levels))
    w = c16[idx] * np.repeat(oenc.fp16_value(scales), group, axis=-1)
    return fp16(w) if rounded_products else w


def sharp_reference(w16, xr, K):
    """(y, bound) for pre-rotated +-1 inputs xr [n][K] against kernel weights w16 [rows][K]."""
    xr = np.atleast_2d(np.asarray(xr, dtype=np.float64))
    y = xr @ w16.T
    bound = acc_depth(K) * 2.0 ** -24 * (np.abs(xr) @ np.abs(w16).T)
    return y, bound
