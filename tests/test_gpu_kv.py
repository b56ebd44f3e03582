"""KV-cache compression on the GPU against the oracle ("How it works", "The KV cache": the
weights' rotation and codebook, 8-bit keys and 3-bit values; "your SSD is a GPU": rotate,
quantize, store, dequantize, de-rotate): the store side is tq_encode with 256 levels (or 8)
on rows of head_dim, checked code by code; the fetch side is tq_kv_fetch, checked against
the oracle's dequantize-and-unrotate on the GPU's own codes, and end to end against the
original rows at the codebook's distortion."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from oracle import codebook as ocb
from oracle import encode as oenc
from parity import as_f64, check_codes, check_scales, torch_to_np
from test_gpu_encode import to_dev

pytestmark = pytest.mark.gpu
OUT_ROUND = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def keys(d, tokens=40, heads=4, dtype=torch.bfloat16, seed=0):
    return to_dev(wl.kv_rows(wl.rng(990, d, seed), tokens, heads, d), dtype)


@pytest.mark.parametrize("d", [64, 128, 256, 1024, 4096])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_store_8bit_keys(d, dtype):
    X = keys(d, dtype=dtype)
    group = 64 if d >= 64 else d
    qw = tq.encode(X, 256, group, seed=4)
    torch.cuda.synchronize()
    ref = oenc.encode(as_f64(X), 256, group, 4)
    rows = X.shape[0]
    assert qw.codes.shape[-1] == d // 4
    check_codes(torch_to_np(qw.codes).reshape(rows, -1), ref, 256, d, f"d {d}")
    check_scales(torch_to_np(qw.scales).reshape(rows, -1), ref, f"d {d}")


def fetch_bound(codes, scales, levels, group, d, ref, odt):
    # fp32 products and log2(d) butterfly stages: (log2 d + 3) 2^-24 ||w'_hat||_1 / sqrt(d)
    # per row, plus the one rounding to the output type
    w = oenc.dequant(codes, scales, levels, group, d)
    lg = int(np.log2(d))
    row = (lg + 3) * 2.0 ** -24 * np.sum(np.abs(w), axis=1, keepdims=True) / np.sqrt(d)
    return row + OUT_ROUND[odt] * np.abs(ref)


@pytest.mark.parametrize("levels", [256, 8, 16, 4])
@pytest.mark.parametrize("group", [16, 32, 64, 128])
@pytest.mark.parametrize("d", [64, 128, 512, 2048])
def test_fetch_matches_oracle(levels, group, d):
    if group > d:
        pytest.skip("group larger than the row")
    odt = [torch.float32, torch.bfloat16, torch.float16][(levels + group + d) % 3]
    X = keys(d, tokens=23, heads=3, seed=levels)
    qw = tq.encode(X, levels, group, seed=7)
    out = tq.kv_fetch(qw, out_dtype=odt)
    torch.cuda.synchronize()
    rows = X.shape[0]
    codes = torch_to_np(qw.codes).reshape(rows, -1)
    scales = torch_to_np(qw.scales).reshape(rows, -1)
    ref = oenc.kv_fetch(codes, scales, levels, group, d, 7)
    got = as_f64(out).reshape(rows, d)
    bound = fetch_bound(codes, scales, levels, group, d, ref, odt)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / bound))


@pytest.mark.parametrize("levels", [256, 8])
def test_round_trip_error_is_the_codebook_distortion(levels):
    # 8-bit keys and 3-bit values of 2048 tokens x 8 heads x 128: the relative squared
    # error of fetch(store(x)) equals the oracle's own round trip on the same rows, and is
    # near the codebook's distortion D (about 4.1e-5 for 8 bits, 0.0345 for 3 bits): after
    # the rotation every group is near-Gaussian, outlier channels and all. (Dividing a group
    # of 64 by its own RMS puts it on a sphere, lighter-tailed than N(0,1), which lowers the
    # 8-bit error below D by about an eighth.)
    X = keys(128, tokens=2048, heads=8, seed=1)
    qw = tq.encode(X, levels, 64, seed=3)
    Y = tq.kv_fetch(qw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    x = as_f64(X)
    y = as_f64(Y).reshape(x.shape)
    err = np.sum((y - x) ** 2) / np.sum(x * x)
    sub = slice(0, 2048)
    ref = oenc.encode(x[sub], levels, 64, 3)
    y_or = oenc.kv_fetch(ref.codes, ref.scales, levels, 64, 128, 3)
    err_or = np.sum((y_or - x[sub]) ** 2) / np.sum(x[sub] ** 2)
    err_sub = np.sum((y[sub] - x[sub]) ** 2) / np.sum(x[sub] ** 2)
    assert abs(err_sub / err_or - 1.0) < 1e-3, (err_sub, err_or)
    D = ocb.distortion(levels)
    assert 0.8 * D < err < 1.05 * D, (err, D)
    # without the rotation the same snap would face the outlier channels: the raw rows'
    # kurtosis is far above a Gaussian's 3, the rotated rows' is close to it
    from oracle import hadamard as ohd
    kurt = lambda a: float(np.mean(a ** 4) / np.mean(a ** 2) ** 2)
    assert kurt(x[:2048]) > 20 and abs(kurt(ohd.rotate(x[:2048], 3)) - 3.0) < 0.2


def test_fetch_of_an_expert_shaped_cache():
    # E x N rows (layers x tokens*heads) are fetched as one block in order
    X = keys(256, tokens=10, heads=2).view(4, 5, 256)
    qw = tq.encode(X, 256, 32, seed=2)
    out = tq.kv_fetch(qw, out_dtype=torch.float32)
    flat = tq.kv_fetch(tq.QWeight(qw.codes.view(1, 20, -1), qw.scales.view(1, 20, -1), qw.signs,
                                  256, 32, 256, 20, 1, 2), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert out.shape == (4, 5, 256) and torch.equal(out.view(20, 256), flat.view(20, 256))
