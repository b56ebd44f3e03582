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
"""

import numpy as np

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
