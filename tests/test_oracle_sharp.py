"""Pins of the sharper output checks in tests/parity.py (no GPU).

* kernel_weights (the decoded weights as the kernels multiply them) differs from the
  oracle's fp64 dequantization by the documented fp16 roundings only: at most 2^-11 of each
  weight, twice that with the rounded matrix-core products.
* The +-1-input check is sharp: one code changed to a neighbouring level anywhere in a row
  moves that row's output by more than the check's bound, at every shape the GPU tests use.
* The a-priori bound holds for an emulation of the kernels' arithmetic (x' rounded to
  fp16 under a power-of-two scale, fp16 centroids and products, fp32 sums in order).
"""

import numpy as np
import pytest

import workloads as wl
from oracle import encode as oenc
from oracle import hadamard as ohd
from parity import acc_depth, apriori_bound, fp16, kernel_weights, sharp_reference

# (levels, group, K): the long rows of the five workloads and the longest 4-bit row the
# sharp GPU tests use
SHAPES = [(8, 128, 4096), (4, 64, 7168), (16, 64, 2048), (3, 16, 2048), (3, 16, 768),
          (16, 128, 4096), (16, 128, 1536), (16, 32, 6144), (3, 32, 7168)]


def encoded(levels, group, K, rows, seed=0):
    W = wl.student_rows(wl.rng(950, levels, K), rows, K).astype(np.float64)
    return oenc.encode(W, levels, group, seed)


@pytest.mark.parametrize("levels,group,K", SHAPES[:4])
@pytest.mark.parametrize("rounded", [False, True])
def test_kernel_weights_within_fp16_rounding_of_dequant(levels, group, K, rounded):
    e = encoded(levels, group, K, 6)
    w16 = kernel_weights(e.codes, e.scales, levels, group, K, rounded)
    w = oenc.dequant(e.codes, e.scales, levels, group, K)
    rel = (2.0 if rounded else 1.0) * 2.0 ** -11
    assert np.all(np.abs(w16 - w) <= rel * np.abs(w) + 1e-300)
    # the roundings are real: the model is not the fp64 dequantization itself
    assert np.any(w16 != w)


def flip_one_per_row(codes, levels, K, g):
    """Each row with one index moved to a neighbouring level at a random position."""
    idx = oenc.unpack(codes, levels, K).copy()
    rows = idx.shape[0]
    pos = g.integers(0, K, rows)
    for r, j in enumerate(pos):
        v = idx[r, j]
        idx[r, j] = v + 1 if v + 1 < levels else v - 1
    return oenc.pack(idx, levels), pos


@pytest.mark.parametrize("levels,group,K", SHAPES)
@pytest.mark.parametrize("rounded", [False, True])
def test_sharp_check_catches_one_wrong_code(levels, group, K, rounded):
    g = wl.rng(951, levels, K)
    e = encoded(levels, group, K, 24)
    w16 = kernel_weights(e.codes, e.scales, levels, group, K, rounded)
    xr = g.choice([-1.0, 1.0], size=(3, K))
    y, bound = sharp_reference(w16, xr, K)
    bad_codes, pos = flip_one_per_row(e.codes, levels, K, g)
    y_bad = xr @ kernel_weights(bad_codes, e.scales, levels, group, K, rounded).T
    # every row of every input is off by more than its bound
    assert np.all(np.abs(y_bad - y) > bound), float(np.min(np.abs(y_bad - y) / bound))


def emulate_kernel(codes, scales, levels, group, K, seed, x, rounded):
    """The kernels' documented arithmetic in numpy: x' = R x (fp64, then rounded to fp16
    after a power-of-two scale that puts max |x'| just under 2^15), weights from
    kernel_weights, products exact, sums in float32 in element order."""
    xr = ohd.rotate(x, seed)
    mx = np.max(np.abs(xr))
    sc = 2.0 ** (14 - np.floor(np.log2(mx)))
    xh = fp16(xr * sc)
    w16 = kernel_weights(codes, scales, levels, group, K, rounded)
    out = np.zeros(w16.shape[0])
    for i in range(w16.shape[0]):
        acc = np.float32(0.0)
        for t in (w16[i] * xh).astype(np.float32):  # products of fp16 values are exact
            acc = np.float32(acc + t)
        out[i] = float(acc) / sc
    return out


@pytest.mark.parametrize("levels,group,K", [(8, 128, 1024), (3, 16, 768), (4, 64, 1536)])
@pytest.mark.parametrize("rounded", [False, True])
def test_apriori_bound_holds_for_emulated_kernel(levels, group, K, rounded):
    g = wl.rng(952, levels, K)
    e = encoded(levels, group, K, 8, seed=3)
    x = wl.gaussian(g, 1, K, outliers=4)[0].astype(np.float64)
    want = (ohd.rotate(x, 3) @ oenc.dequant(e.codes, e.scales, levels, group, K).T)
    got = emulate_kernel(e.codes, e.scales, levels, group, K, 3, x, rounded)
    bound = apriori_bound(e.codes, e.scales, levels, group, K, 3, x)
    assert np.all(np.abs(got - want) <= bound)
    # and the emulated error is not negligible next to it: the bound is within 200x
    assert np.max(np.abs(got - want) / bound) > 5e-3


def test_depth_allows_the_longest_matrix_core_chain():
    # K/16 matrix instructions along K plus a DPP/LDS reduction tree of at most 64 adds
    for K in (64, 768, 4096, 8192):
        assert acc_depth(K) >= K // 16 + 6
