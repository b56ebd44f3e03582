"""Sharp parity of the qmv family on long rows: pre-rotated inputs of +-1 (exact in every
input dtype and in the kernels' scaled fp16), compared with the decoded weights as the
kernels multiply them (tests/parity.py kernel_weights). The only error left is the fp32
summation, so one wrong code anywhere in a row fails the check (tests/test_oracle_sharp.py
plants such flips at these shapes). Through the C ABI, on the GPU's own codes."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from parity import as_f64, check_outputs, kernel_weights, sharp_reference, torch_to_np
from test_gpu_encode import to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(8, 128, 4096), (4, 64, 7168), (16, 64, 2048), (3, 16, 2048), (3, 16, 768),
          (16, 128, 4096), (16, 128, 1536), (16, 32, 6144), (3, 32, 7168)]
XDT = [torch.bfloat16, torch.float16, torch.float32]


def stack(levels, group, K, E, N, seed):
    g = wl.rng(970, levels, K)
    W = to_dev(wl.student_rows(g, E * N, K), torch.bfloat16).view(E, N, K)
    qw = tq.encode(W, levels, group, seed)
    torch.cuda.synchronize()
    codes = torch_to_np(qw.codes).reshape(E, N, -1)
    scales = torch_to_np(qw.scales).reshape(E, N, -1)
    return qw, codes, scales


def pm1(g, n, K, dtype):
    xr = g.choice([-1.0, 1.0], size=(n, K))
    return xr, torch.from_numpy(xr).to(dtype).cuda()


@pytest.mark.parametrize("levels,group,K", SHAPES)
def test_qmv_and_gather_qmv_pm1(levels, group, K):
    E, N = 5, 48
    qw, codes, scales = stack(levels, group, K, E, N, 11)
    g = wl.rng(971, levels, K)
    for i, xdt in enumerate(XDT):
        xr, x = pm1(g, 1, K, xdt)
        e = i % E
        y = tq.qmv(qw.expert(e), x[0], rotated=True)
        ids_np = np.array([4, 0, 2, 2, 1, 3][: 3 + i], dtype=np.int32)
        yg = tq.gather_qmv(qw, torch.from_numpy(ids_np).cuda(), x[0], rotated=True)
        torch.cuda.synchronize()
        w16 = kernel_weights(codes[e], scales[e], levels, group, K, False)
        want, bound = sharp_reference(w16, xr, K)
        check_outputs(as_f64(y)[None], want, bound, f"qmv expert {e} x {xdt}")
        ygf = as_f64(yg)
        for k, ek in enumerate(ids_np):
            w16 = kernel_weights(codes[ek], scales[ek], levels, group, K, False)
            want, bound = sharp_reference(w16, xr, K)
            check_outputs(ygf[k][None], want, bound, f"gather_qmv slot {k} expert {ek}")


@pytest.mark.parametrize("levels,group,K", SHAPES)
def test_multi_gather_qmv_pm1(levels, group, K):
    E, N, P = 5, 40, 21
    qw, codes, scales = stack(levels, group, K, E, N, 12)
    g = wl.rng(972, levels, K)
    ids_np = g.integers(0, E, P).astype(np.int32)
    ids_np[:3] = 1  # one expert with several pairs
    xr, X = pm1(g, P, K, torch.bfloat16)
    y = tq.multi_gather_qmv(qw, torch.from_numpy(ids_np).cuda(), X, rotated=True)
    torch.cuda.synchronize()
    yg = as_f64(y)
    for p_, e in enumerate(ids_np):
        w16 = kernel_weights(codes[e], scales[e], levels, group, K, True)
        want, bound = sharp_reference(w16, xr[p_], K)
        check_outputs(yg[p_][None], want, bound, f"pair {p_} expert {e}")


@pytest.mark.parametrize("levels,group,K", SHAPES)
def test_gather_qmm_pm1(levels, group, K):
    E, N, T = 5, 80, 24
    qw, codes, scales = stack(levels, group, K, E, N, 13)
    g = wl.rng(973, levels, K)
    counts = np.array([9, 0, 33, 1, 12])  # an empty expert, a single row, a partial tile
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offsets[-1])
    row_token = g.integers(0, T, M).astype(np.int32)
    xr, X = pm1(g, T, K, torch.float16)
    y = tq.gather_qmm(qw, X, torch.from_numpy(row_token).cuda(), torch.from_numpy(offsets).cuda(),
                      rotated=True)
    torch.cuda.synchronize()
    yg = as_f64(y)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b == a:
            continue
        w16 = kernel_weights(codes[e], scales[e], levels, group, K, True)
        want, bound = sharp_reference(w16, xr[row_token[a:b]], K)
        check_outputs(yg[a:b], want, bound, f"gather_qmm expert {e}")
