"""The dense-rotation path on the GPU (VeloxQuant-MLX's QR-derived rotation for input
dimensions the Hadamard transform does not cover, such as 4864), through the C ABI:
tq_rotate_dense against the oracle's R x, tq_encode_dense code for code against the
oracle's encode_dense, and the qmv family, dequant and gather_qmm at K = 4864 on inputs
rotated by tq_rotate_dense, against the oracle's dequantize-then-multiply."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from oracle import encode as oenc
from oracle import ops as oops
from parity import (as_f64, check_codes, check_outputs, check_scales, kernel_weights,
                    sharp_reference, torch_to_np)
from test_gpu_encode import to_dev

pytestmark = pytest.mark.gpu
OUT_ROUND = {torch.float32: 2.0 ** -24, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


def rot(K, seed=1):
    R = wl.haar_rotation(K, seed)
    return R, torch.from_numpy(np.array(R)).cuda()


@pytest.mark.parametrize("K,rows", [(4864, 1), (4864, 3), (4864, 70), (160, 130), (640, 65), (640, 8)])
@pytest.mark.parametrize("xdt,odt", [(torch.bfloat16, torch.float32), (torch.float32, torch.float32),
                                     (torch.float16, torch.bfloat16)])
def test_rotate_dense(K, rows, xdt, odt):
    R, Rd = rot(K)
    x = to_dev(wl.gaussian(wl.rng(1000, K, rows), rows, K, outliers=4), xdt)
    y = tq.rotate_dense(x, Rd, out_dtype=odt)
    torch.cuda.synchronize()
    ref = oops.rotate_dense(as_f64(x), R)
    # exact products, fp64 sums: only the one rounding to the output type is left
    tol = OUT_ROUND[odt] * np.abs(ref) + 1e-12 * np.linalg.norm(as_f64(x), axis=1, keepdims=True)
    assert np.all(np.abs(as_f64(y) - ref) <= tol)


@pytest.mark.parametrize("levels,group", [(8, 128), (3, 16), (16, 64), (4, 32)])
@pytest.mark.parametrize("ws_rows", [None, 7])
def test_encode_dense_matches_oracle(levels, group, ws_rows):
    K, rows = 4864, 40
    R, Rd = rot(K, 2)
    W = to_dev(wl.student_rows(wl.rng(1001, levels, group), rows, K), torch.bfloat16)
    kw = {} if ws_rows is None else {"ws_bytes": ws_rows * K * 8}  # several chunks
    qw = tq.encode_dense(W, Rd, levels, group, **kw)
    torch.cuda.synchronize()
    ref = oenc.encode_dense(as_f64(W), R, levels, group)
    check_codes(torch_to_np(qw.codes).reshape(rows, -1), ref, levels, K, "dense")
    check_scales(torch_to_np(qw.scales).reshape(rows, -1), ref, "dense")


def dense_reference(codes, scales, levels, group, K, R, X):
    """(y, bound): the oracle's product with the dense rotation and the smaller of the
    required bound and the a-priori rounding bound of tests/parity.py."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    Wq = oenc.dequant(codes, scales, levels, group, K)
    xr = oops.rotate_dense(X, R)
    y = xr @ Wq.T
    req = 2e-3 * np.multiply.outer(np.linalg.norm(X, axis=1), np.linalg.norm(Wq, axis=1))
    rel = 3.0 * 2.0 ** -11 + (K // 16 + 64) * 2.0 ** -24
    apri = rel * (np.abs(xr) @ np.abs(Wq).T) + 2.0 ** -16 * np.multiply.outer(
        np.linalg.norm(X, axis=1), np.sum(np.abs(Wq), axis=1))
    return y, np.minimum(req, apri)


@pytest.mark.parametrize("levels,group", [(8, 128), (3, 16), (4, 64)])
def test_layers_at_k_4864_with_a_dense_rotation(levels, group):
    K, N, E = 4864, 96, 3
    R, Rd = rot(K, 3)
    g = wl.rng(1002, levels, group)
    W = to_dev(wl.student_rows(g, E * N, K), torch.bfloat16).view(E, N, K)
    qw = tq.encode_dense(W, Rd, levels, group)
    codes = torch_to_np(qw.codes).reshape(E, N, -1)
    scales = torch_to_np(qw.scales).reshape(E, N, -1)
    # one token: qmv and gather_qmv on R x
    x = to_dev(wl.gaussian(g, 1, K, outliers=4)[0], torch.bfloat16)
    xr = tq.rotate_dense(x.view(1, K), Rd).view(K)
    y = tq.qmv(qw.expert(1), xr, rotated=True)
    ids = np.array([2, 0, 2], dtype=np.int32)
    yg = tq.gather_qmv(qw, torch.from_numpy(ids).cuda(), xr, rotated=True)
    # prefill pairs and a sorted batch
    P = 12
    X = to_dev(wl.gaussian(g, P, K), torch.bfloat16)
    XR = tq.rotate_dense(X, Rd)
    pids = g.integers(0, E, P).astype(np.int32)
    ym = tq.multi_gather_qmv(qw, torch.from_numpy(pids).cuda(), XR, rotated=True)
    counts = np.array([5, 0, 7])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rt = g.integers(0, P, int(off[-1])).astype(np.int32)
    yq = tq.gather_qmm(qw, XR, torch.from_numpy(rt).cuda(), torch.from_numpy(off).cuda(), rotated=True)
    deq = tq.dequant(qw, out_dtype=torch.float32)
    torch.cuda.synchronize()
    xf, Xf = as_f64(x), as_f64(X)
    want, bound = dense_reference(codes[1], scales[1], levels, group, K, R, xf)
    check_outputs(as_f64(y)[None], want, bound, "qmv")
    for k, e in enumerate(ids):
        want, bound = dense_reference(codes[e], scales[e], levels, group, K, R, xf)
        check_outputs(as_f64(yg[k])[None], want, bound, f"gather_qmv {k}")
    for p_, e in enumerate(pids):
        want, bound = dense_reference(codes[e], scales[e], levels, group, K, R, Xf[p_])
        check_outputs(as_f64(ym[p_])[None], want, bound, f"multi_gather {p_}")
    for e in range(E):
        a, b = off[e], off[e + 1]
        if b > a:
            want, bound = dense_reference(codes[e], scales[e], levels, group, K, R, Xf[rt[a:b]])
            check_outputs(as_f64(yq[a:b]), want, bound, f"gather_qmm expert {e}")
    ref = oenc.dequant(codes.reshape(E * N, -1), scales.reshape(E * N, -1), levels, group, K)
    got = as_f64(deq).reshape(E * N, K)
    assert np.all(np.abs(got - ref) <= 2.0 ** -23 * np.abs(ref))


@pytest.mark.parametrize("levels,group", [(16, 64), (3, 16)])
def test_sharp_decode_at_k_4864(levels, group):
    # +-1 pre-rotated inputs: any wrong code in a 4864-long row shows (tests/parity.py)
    K, N = 4864, 64
    R, Rd = rot(K, 4)
    g = wl.rng(1003, levels)
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    qw = tq.encode_dense(W, Rd, levels, group)
    xr = g.choice([-1.0, 1.0], size=(1, K))
    y = tq.qmv(qw, torch.from_numpy(xr[0]).to(torch.bfloat16).cuda(), rotated=True)
    X = g.choice([-1.0, 1.0], size=(8, K))
    off = torch.tensor([0, 8], dtype=torch.int32, device="cuda")
    yq = tq.gather_qmm(qw, torch.from_numpy(X).to(torch.float16).cuda(),
                       torch.arange(8, dtype=torch.int32, device="cuda"), off, rotated=True)
    torch.cuda.synchronize()
    codes, scales = torch_to_np(qw.codes).reshape(N, -1), torch_to_np(qw.scales).reshape(N, -1)
    want, bound = sharp_reference(kernel_weights(codes, scales, levels, group, K, False), xr, K)
    check_outputs(as_f64(y)[None], want, bound, "qmv +-1")
    want, bound = sharp_reference(kernel_weights(codes, scales, levels, group, K, True), X, K)
    check_outputs(as_f64(yq), want, bound, "gather_qmm +-1")
