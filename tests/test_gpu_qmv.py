"""GPU parity of the qmv family (tq_qmv, tq_gather_qmv, tq_multi_gather_qmv, tq_gather_qmm)
against the oracle's dequantize-then-multiply in fp64, through the C ABI."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from oracle import encode as oenc
from oracle import hadamard as ohd
from oracle import ops as oops
from parity import as_f64, check_codes, check_outputs, qmv_reference, torch_to_np
from test_gpu_encode import to_dev

pytestmark = pytest.mark.gpu


def encode_both(W_dev, levels, group, seed):
    """GPU encode, and the oracle's encode of the same bytes."""
    qw = tq.encode(W_dev, levels, group, seed)
    torch.cuda.synchronize()
    rows = W_dev.numel() // W_dev.shape[-1]
    ref = oenc.encode(as_f64(W_dev).reshape(rows, -1), levels, group, seed)
    return qw, ref


def gpu_arrays(qw):
    E = qw.E
    return (torch_to_np(qw.codes).reshape(E, qw.N, -1), torch_to_np(qw.scales).reshape(E, qw.N, -1))


def check_qmv_against_oracle(qw, ref, x_dev, y, tag):
    codes, scales = gpu_arrays(qw)
    x = as_f64(x_dev)
    yg = as_f64(y)
    want, bound = qmv_reference(codes[0], scales[0], qw.levels, qw.group, qw.K, qw.seed, x)
    worst = check_outputs(yg, want, bound, tag + " (GPU codes)")
    want2, bound2 = qmv_reference(ref.codes, ref.scales, qw.levels, qw.group, qw.K, qw.seed, x)
    check_outputs(yg, want2, bound2, tag + " (oracle codes)")
    return worst


def test_single_layer_end_to_end():
    # 256 x 512 fp32 weight, rotation signs from seed 0, 4-bit Lloyd-Max, group 64; one
    # fp32 activation; the result equals dequantize-then-multiply
    c = wl.C1
    p = c.projs[0]
    W = torch.from_numpy(wl.student_rows(wl.rng(c.cid, wl.T_W), p.N, p.K)).cuda()
    x = torch.from_numpy(wl.gaussian(wl.rng(c.cid, wl.T_X), 1, p.K)[0]).cuda()
    qw, ref = encode_both(W, p.levels, p.group, p.seed)
    assert check_codes(torch_to_np(qw.codes).reshape(p.N, -1), ref, p.levels, p.K) == 0
    y = tq.qmv(qw, x)
    torch.cuda.synchronize()
    check_qmv_against_oracle(qw, ref, x, y, "C1")
    # brute force in the original basis: (R^T w'_hat) . x
    yb = oops.qmv_unrotated(ref.codes, ref.scales, p.levels, p.group, p.K, p.seed, as_f64(x))
    b = oops.row_bound(ref.codes, ref.scales, p.levels, p.group, p.K, as_f64(x))
    check_outputs(as_f64(y), yb, b, "C1 unrotated")


def test_dense_decode_full_size():
    # 4096 x 4096 bf16, 3-bit g128, bf16 activation with 8 outlier channels x20
    c = wl.C2
    p = c.projs[0]
    W = to_dev(wl.student_rows(wl.rng(c.cid, wl.T_W), p.N, p.K), torch.bfloat16)
    x = to_dev(wl.gaussian(wl.rng(c.cid, wl.T_X), 1, p.K, outliers=8)[0], torch.bfloat16)
    qw, ref = encode_both(W, p.levels, p.group, p.seed)
    n = check_codes(torch_to_np(qw.codes).reshape(p.N, -1), ref, p.levels, p.K, "C2")
    assert n <= 16
    y = tq.qmv(qw, x)
    torch.cuda.synchronize()
    check_qmv_against_oracle(qw, ref, x, y, "C2")


FORMATS = [(L, g) for L in (3, 4, 8, 16) for g in (16, 32, 64, 128)]


@pytest.mark.parametrize("levels,group", FORMATS)
@pytest.mark.parametrize("K,N", [(1536, 200), (640, 77), (7168, 64), (2048, 300), (6144, 40)])
def test_qmv_formats(levels, group, K, N):
    g = wl.rng(910, levels * 1000 + group, K)
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    x = to_dev(wl.gaussian(g, 1, K, outliers=4)[0], torch.bfloat16)
    qw, ref = encode_both(W, levels, group, seed=11)
    y = tq.qmv(qw, x)
    torch.cuda.synchronize()
    check_qmv_against_oracle(qw, ref, x, y, f"L{levels} g{group} K{K} N{N}")


@pytest.mark.parametrize("levels", [3, 4, 8, 16])
@pytest.mark.parametrize("K", [64, 96, 128, 256, 224, 8192])
def test_qmv_small_and_largest_k(levels, K):
    # few chunks per row (2..13: lanes of a wave split over several rows) and the largest K
    group = 16 if K % 32 else 32
    N = 70
    g = wl.rng(920, levels, K)
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    x = to_dev(wl.gaussian(g, 1, K)[0], torch.float32)
    qw, ref = encode_both(W, levels, group, seed=13)
    y = tq.qmv(qw, x)
    torch.cuda.synchronize()
    check_qmv_against_oracle(qw, ref, x, y, f"L{levels} K{K}")


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16, torch.float16])
def test_qmv_dtypes(xdt, ydt):
    K, N, levels, group = 768, 130, 8, 32
    g = wl.rng(911, 0)
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    x = to_dev(wl.gaussian(g, 1, K)[0], xdt)
    qw, ref = encode_both(W, levels, group, seed=2)
    y = tq.qmv(qw, x, out_dtype=ydt)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    want, bound = qmv_reference(codes[0], scales[0], levels, group, K, 2, as_f64(x))
    out_round = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}[ydt]
    check_outputs(as_f64(y), want, bound + out_round * np.abs(want), f"x {xdt} y {ydt}")


def test_qmv_pre_rotated_input():
    K, N, levels, group = 1536, 96, 16, 64
    g = wl.rng(912, 0)
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    x = wl.gaussian(g, 1, K)[0].astype(np.float64)
    xr = torch.from_numpy(ohd.rotate(x, 4).astype(np.float32)).cuda()
    qw, ref = encode_both(W, levels, group, seed=4)
    y = tq.qmv(qw, xr, rotated=True)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    want, bound = qmv_reference(codes[0], scales[0], levels, group, K, 4, x)
    check_outputs(as_f64(y), want, bound + 1e-6 * np.abs(want), "rotated input")


def test_qmv_large_input_and_zero_input():
    K, N, levels, group = 512, 64, 16, 64
    g = wl.rng(913, 0)
    W = to_dev(wl.student_rows(g, N, K), torch.float32)
    qw, ref = encode_both(W, levels, group, seed=0)
    for scale in (1e-30, 1e4, 1e30):
        x = torch.from_numpy(wl.gaussian(g, 1, K)[0] * np.float32(scale)).cuda()
        y = tq.qmv(qw, x)
        torch.cuda.synchronize()
        check_qmv_against_oracle(qw, ref, x, y, f"x*{scale}")
    y = tq.qmv(qw, torch.zeros(K, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(y == 0)


@pytest.mark.parametrize("levels", [4, 8, 16])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16])
def test_qmv_k4096_16bit_inputs(levels, xdt):
    # K = 4096 with a 16-bit input takes the matrix-core rotation: every bit format, both
    # 16-bit types, inputs far from 1 in both directions (bf16 only: fp16 cannot hold them)
    # and the zero input
    K, N, group = 4096, 96, 64
    g = wl.rng(915, levels, int(xdt == torch.float16))
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    qw, ref = encode_both(W, levels, group, seed=5)
    scales = (1.0, 2.0 ** -100, 2.0 ** 100) if xdt == torch.bfloat16 else (1.0, 2.0 ** -10, 2.0 ** 10)
    for sc in scales:
        x = to_dev(wl.gaussian(g, 1, K, outliers=8)[0] * sc, xdt)
        y = tq.qmv(qw, x)
        torch.cuda.synchronize()
        check_qmv_against_oracle(qw, ref, x, y, f"L{levels} {xdt} x*{sc}")
    y = tq.qmv(qw, torch.zeros(K, dtype=xdt, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(y == 0)


@pytest.mark.parametrize("levels", [4, 8, 16])
@pytest.mark.parametrize("K,N,xdt", [(2048, 333, torch.float32), (4096, 250, torch.bfloat16),
                                     (4096, 77, torch.float16), (8192, 96, torch.bfloat16),
                                     (2048, 1000, torch.float16)])
def test_qmv_power_of_two_k_group_128(levels, K, N, xdt):
    # groups of 128 with K in {2048, 4096, 8192}: every bit format and input type, row counts
    # that are not a multiple of the rows a workgroup takes
    g = wl.rng(916, levels, K + N)
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    qw, ref = encode_both(W, levels, 128, seed=6)
    x = to_dev(wl.gaussian(g, 1, K, outliers=4)[0], xdt)
    y = tq.qmv(qw, x)
    torch.cuda.synchronize()
    check_qmv_against_oracle(qw, ref, x, y, f"L{levels} K{K} N{N} {xdt}")


def test_gather_qmv_k4096_bad_ids():
    # several experts at K = 4096 (rotation on the matrix cores), slots with ids out of range
    # (NaN rows)
    E, N, K, levels = 5, 40, 4096, 8
    qw, ref = make_experts(917, E, N, K, levels, 128, seed=3)
    ids_np = np.array([4, 0, E, 2, -1, 1], dtype=np.int32)
    x = to_dev(wl.gaussian(wl.rng(917, 1), 1, K)[0], torch.bfloat16)
    y = tq.gather_qmv(qw, torch.from_numpy(ids_np).cuda(), x)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    yg, xf = as_f64(y), as_f64(x)
    for k, e in enumerate(ids_np):
        if 0 <= e < E:
            want, bound = qmv_reference(codes[e], scales[e], levels, 128, K, 3, xf)
            check_outputs(yg[k], want, bound, f"slot {k} expert {e}")
        else:
            assert np.all(np.isnan(yg[k])), k


def make_experts(cfg, E, N, K, levels, group, seed, dtype=torch.bfloat16):
    W = torch.stack([to_dev(wl.student_rows(wl.rng(cfg, 20, e), N, K), dtype) for e in range(E)])
    return encode_both(W, levels, group, seed)


@pytest.mark.parametrize("levels,group,K,N", [(4, 64, 7168, 96), (16, 64, 2048, 160),
                                              (3, 16, 768, 64), (8, 128, 4096, 64)])
def test_gather_qmv(levels, group, K, N):
    E = 9
    qw, ref = make_experts(914, E, N, K, levels, group, seed=0)
    x = to_dev(wl.gaussian(wl.rng(914, 1), 1, K)[0], torch.bfloat16)
    ids = torch.tensor([3, 8, 0, 3, 5, 1, 7, 2], dtype=torch.int32, device="cuda")
    y = tq.gather_qmv(qw, ids, x)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    yg = as_f64(y)
    for k, e in enumerate(ids.tolist()):
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 0, as_f64(x))
        check_outputs(yg[k], want, bound, f"slot {k} expert {e}")
    # each slot equals a dense qmv on that expert's weights
    y0 = tq.qmv(qw.expert(3), x)
    torch.cuda.synchronize()
    assert torch.equal(y0, y[0]) and torch.equal(y0, y[3])


@pytest.mark.parametrize("levels,group,K,N,xdt,rotated",
                         [(4, 64, 7168, 96, torch.bfloat16, False), (3, 16, 768, 64, torch.float16, False),
                          (8, 128, 4096, 40, torch.bfloat16, False), (16, 64, 2048, 72, torch.float32, True)])
def test_gather_qmv_pair(levels, group, K, N, xdt, rotated):
    # gate and up in one launch: rows k from the first weight, rows n + k from the second,
    # each equal to its own gather_qmv call bit for bit and to the oracle within the bound
    E = 7
    g1, _ = make_experts(930, E, N, K, levels, group, seed=5)
    W2 = torch.stack([to_dev(wl.student_rows(wl.rng(931, 20, e), N, K), torch.bfloat16)
                      for e in range(E)])
    g2, _ = encode_both(W2, levels, group, 5)
    ids_np = np.array([6, 0, 3, 3, E, 2, -2, 5], dtype=np.int32)
    ids = torch.from_numpy(ids_np).cuda()
    x0 = wl.gaussian(wl.rng(930, 1), 1, K)[0]
    if rotated:
        # the oracle rotates the original input; the kernel takes R x in fp32
        xf = x0.astype(np.float64)
        x = torch.from_numpy(ohd.rotate(xf, 5).astype(np.float32)).cuda()
        extra = 1e-6
    else:
        x = to_dev(x0, xdt)
        xf = as_f64(x)
        extra = 0.0
    with pytest.raises(ValueError):  # an output buffer one row short is refused
        tq.gather_qmv_pair(g1, g2, ids, x, rotated=rotated,
                           out=torch.empty((2 * len(ids_np) - 1, N), device="cuda"))
    y = tq.gather_qmv_pair(g1, g2, ids, x, rotated=rotated)
    y1 = tq.gather_qmv(g1, ids, x, rotated=rotated)
    y2 = tq.gather_qmv(g2, ids, x, rotated=rotated)
    torch.cuda.synchronize()
    n = len(ids_np)
    assert y.shape == (2 * n, N)
    assert torch.equal(torch.nan_to_num(y[:n], nan=7.0), torch.nan_to_num(y1, nan=7.0))
    assert torch.equal(torch.nan_to_num(y[n:], nan=7.0), torch.nan_to_num(y2, nan=7.0))
    yg = as_f64(y)
    for half, qw in ((0, g1), (1, g2)):
        codes, scales = gpu_arrays(qw)
        for k, e in enumerate(ids_np):
            row = yg[half * n + k]
            if 0 <= e < E:
                want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 5, xf)
                check_outputs(row, want, bound + extra * np.abs(want),
                              f"weight {half} slot {k} expert {e}")
            else:
                assert np.all(np.isnan(row)), (half, k)


def test_gather_qmv_bad_id_gives_nan_rows():
    K, N, levels, group = 512, 40, 16, 64
    qw, _ = make_experts(915, 3, N, K, levels, group, seed=0)
    x = to_dev(wl.gaussian(wl.rng(915, 1), 1, K)[0], torch.bfloat16)
    ids = torch.tensor([1, 3, -1, 0], dtype=torch.int32, device="cuda")
    y = tq.gather_qmv(qw, ids, x)
    torch.cuda.synchronize()
    assert torch.isnan(y[1]).all() and torch.isnan(y[2]).all()
    assert torch.isfinite(y[0]).all() and torch.isfinite(y[3]).all()


@pytest.mark.parametrize("levels,group,K,N", [(3, 16, 2048, 96), (3, 16, 768, 160),
                                              (3, 16, 2048, 33), (3, 16, 1280, 72),
                                              (3, 32, 2560, 136), (3, 64, 1280, 64),
                                              (3, 128, 1536, 40), (3, 32, 384, 72),
                                              (16, 64, 1536, 64), (4, 32, 7168, 48),
                                              (8, 128, 6144, 40), (4, 64, 5120, 40)])
def test_multi_gather(levels, group, K, N):
    E = 12
    qw, _ = make_experts(916, E, N, K, levels, group, seed=1)
    g = wl.rng(916, 2)
    # skewed pairs: expert 5 gets 19 inputs (three batches), some experts none
    ids = np.concatenate([np.full(19, 5), g.integers(0, E, 30), [11, 0, 0]]).astype(np.int32)
    g.shuffle(ids)
    P = len(ids)
    X = to_dev(wl.gaussian(g, P, K), torch.bfloat16)
    y = tq.multi_gather_qmv(qw, torch.from_numpy(ids).cuda(), X)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    Xf = as_f64(X)
    yg = as_f64(y)
    for p_ in range(P):
        e = ids[p_]
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 1, Xf[p_])
        check_outputs(yg[p_], want, bound, f"pair {p_} expert {e}")


@pytest.mark.parametrize("levels,group,K,N", [(3, 16, 2048, 96), (3, 32, 1280, 136),
                                              (3, 16, 768, 64), (16, 64, 1536, 64)])
def test_multi_gather_pair(levels, group, K, N):
    # gate and up over the same pairs in one call: rows p from the first weight, rows P + p
    # from the second, each equal to its own multi_gather_qmv call bit for bit and to the
    # oracle within the bound; bad pairs give NaN rows in both halves
    E = 9
    g1, _ = make_experts(932, E, N, K, levels, group, seed=2)
    W2 = torch.stack([to_dev(wl.student_rows(wl.rng(933, 20, e), N, K), torch.bfloat16)
                      for e in range(E)])
    g2, _ = encode_both(W2, levels, group, 2)
    g = wl.rng(932, 2)
    ids = np.concatenate([np.full(21, 4), g.integers(0, E, 40), [8, 0, E, -3]]).astype(np.int32)
    g.shuffle(ids)
    P = len(ids)
    X = to_dev(wl.gaussian(g, P, K), torch.bfloat16)
    ids_d = torch.from_numpy(ids).cuda()
    y = tq.multi_gather_qmv_pair(g1, g2, ids_d, X)
    y1 = tq.multi_gather_qmv(g1, ids_d, X)
    y2 = tq.multi_gather_qmv(g2, ids_d, X)
    torch.cuda.synchronize()
    assert y.shape == (2 * P, N)
    assert torch.equal(torch.nan_to_num(y[:P], nan=7.0), torch.nan_to_num(y1, nan=7.0))
    assert torch.equal(torch.nan_to_num(y[P:], nan=7.0), torch.nan_to_num(y2, nan=7.0))
    Xf = as_f64(X)
    yg = as_f64(y)
    for half, qw in ((0, g1), (1, g2)):
        codes, scales = gpu_arrays(qw)
        for p_ in range(P):
            e = ids[p_]
            row = yg[half * P + p_]
            if 0 <= e < E:
                want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 2, Xf[p_])
                check_outputs(row, want, bound, f"weight {half} pair {p_} expert {e}")
            else:
                assert np.all(np.isnan(row)), (half, p_)


def test_multi_gather_bad_ids_and_empty():
    K, N, levels, group = 512, 32, 8, 64
    qw, _ = make_experts(917, 4, N, K, levels, group, seed=0)
    X = to_dev(wl.gaussian(wl.rng(917, 1), 5, K), torch.bfloat16)
    ids = torch.tensor([0, 4, 2, -7, 2], dtype=torch.int32, device="cuda")
    y = tq.multi_gather_qmv(qw, ids, X)
    torch.cuda.synchronize()
    assert torch.isnan(y[1]).all() and torch.isnan(y[3]).all()
    assert torch.isfinite(y[[0, 2, 4]]).all()
    y0 = tq.multi_gather_qmv(qw, ids[:0], X[:0])
    torch.cuda.synchronize()
    assert y0.shape == (0, N)


def routing_case(T, E, k, cfg):
    row_token, row_expert, offsets = wl.zipf_sorted_routing(cfg, T, E, k)
    return row_token, row_expert, offsets


@pytest.mark.parametrize("levels,group,K,N", [(16, 128, 4096, 192), (16, 128, 1536, 320),
                                              (8, 64, 768, 100), (3, 16, 2048, 64),
                                              (4, 32, 640, 130), (16, 64, 6144, 72),
                                              (8, 32, 1280, 90), (16, 32, 96, 40),
                                              (4, 16, 160, 70), (16, 16, 224, 33),
                                              (8, 32, 96, 50), (4, 32, 224, 100),
                                              (3, 16, 7168, 40), (3, 128, 768, 48),
                                              (16, 16, 2048, 80), (8, 16, 5120, 40),
                                              (4, 16, 1536, 64)])
def test_gather_qmm(levels, group, K, N):
    # (K 96, 160, 224: an odd multiple of 32, so the last K step is half empty; trits with
    # 128 and 448 groups per row: the LDS window of staged scales moves along the row;
    # groups of 16 with 96 to 320 groups per row, their scales loaded per lane)
    E, T, k = 10, 96, 3
    qw, _ = make_experts(918, E, N, K, levels, group, seed=2)
    row_token, row_expert, offsets = routing_case(T, E, k, 918 + K)
    X = to_dev(wl.gaussian(wl.rng(918, 3), T, K), torch.bfloat16)
    y = tq.gather_qmm(qw, X, torch.from_numpy(row_token).cuda(), torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    Xf = as_f64(X)
    yg = as_f64(y)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b == a:
            continue
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 2, Xf[row_token[a:b]])
        check_outputs(yg[a:b], want, bound, f"expert {e}")


@pytest.mark.parametrize("levels,group,K,N", [(16, 128, 4096, 192), (3, 16, 2048, 64),
                                              (8, 32, 1280, 90)])
def test_gather_qmm_pair(levels, group, K, N):
    # gate and up over the same sorted rows: rows m from the first weight, rows M + m from
    # the second, each equal to its own gather_qmm call bit for bit and to the oracle within
    # the bound; an out-of-range token gives NaN rows in both halves
    E, T, k = 8, 64, 3
    g1, _ = make_experts(934, E, N, K, levels, group, seed=6)
    W2 = torch.stack([to_dev(wl.student_rows(wl.rng(935, 20, e), N, K), torch.bfloat16)
                      for e in range(E)])
    g2, _ = encode_both(W2, levels, group, 6)
    row_token, _, offsets = routing_case(T, E, k, 934 + K)
    row_token = row_token.copy()
    row_token[5] = T + 3
    M = len(row_token)
    X = to_dev(wl.gaussian(wl.rng(934, 3), T, K), torch.bfloat16)
    rt, off = torch.from_numpy(row_token).cuda(), torch.from_numpy(offsets).cuda()
    y = tq.gather_qmm_pair(g1, g2, X, rt, off)
    y1 = tq.gather_qmm(g1, X, rt, off)
    y2 = tq.gather_qmm(g2, X, rt, off)
    torch.cuda.synchronize()
    assert y.shape == (2 * M, N)
    assert torch.equal(torch.nan_to_num(y[:M], nan=7.0), torch.nan_to_num(y1, nan=7.0))
    assert torch.equal(torch.nan_to_num(y[M:], nan=7.0), torch.nan_to_num(y2, nan=7.0))
    Xf = as_f64(X)
    yg = as_f64(y)
    assert np.isnan(yg[5]).all() and np.isnan(yg[M + 5]).all()
    for half, qw in ((0, g1), (1, g2)):
        codes, scales = gpu_arrays(qw)
        for e in range(E):
            rows = [m for m in range(offsets[e], offsets[e + 1]) if m != 5]
            if not rows:
                continue
            want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 6,
                                        Xf[row_token[rows]])
            check_outputs(yg[half * M + np.array(rows)], want, bound, f"weight {half} expert {e}")


@pytest.mark.parametrize("op", ["multi_gather", "gather_qmm"])
def test_pair_calls_take_pre_rotated_inputs(op):
    # the multi_gather and gather_qmm pairs with inputs already rotated (fp32 R x): no signs
    # are read, and each half matches the oracle on the original inputs
    levels, group, K, N, E = 16, 64, 1536, 48, 5
    g1, _ = make_experts(936, E, N, K, levels, group, seed=3)
    W2 = torch.stack([to_dev(wl.student_rows(wl.rng(937, 20, e), N, K), torch.bfloat16)
                      for e in range(E)])
    g2, _ = encode_both(W2, levels, group, 3)
    g = wl.rng(936, 2)
    rows = 12
    X0 = wl.gaussian(g, rows, K).astype(np.float64)
    Xr = torch.from_numpy(ohd.rotate(X0, 3).astype(np.float32)).cuda()
    if op == "multi_gather":
        ids = g.integers(0, E, rows).astype(np.int32)
        y = tq.multi_gather_qmv_pair(g1, g2, torch.from_numpy(ids).cuda(), Xr, rotated=True)
        experts, xs, n = ids, X0, rows
    else:
        offsets = np.array([0, 3, 3, 8, 10, 12], dtype=np.int32)
        row_token = g.integers(0, rows, 12).astype(np.int32)
        y = tq.gather_qmm_pair(g1, g2, Xr, torch.from_numpy(row_token).cuda(),
                               torch.from_numpy(offsets).cuda(), rotated=True)
        experts = np.repeat(np.arange(E), np.diff(offsets))
        xs, n = X0[row_token], 12
    torch.cuda.synchronize()
    yg = as_f64(y)
    for half, qw in ((0, g1), (1, g2)):
        codes, scales = gpu_arrays(qw)
        for i in range(n):
            e = int(experts[i])
            want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 3, xs[i])
            check_outputs(yg[half * n + i], want, bound + 1e-6 * np.abs(want),
                          f"{op} weight {half} row {i}")


def test_gather_qmm_edges():
    # experts with no rows, an expert with more rows than one tile, rows past the end of N,
    # an out-of-range token id (NaN row), and a pre-rotated bf16 input
    K, N, levels, group = 512, 70, 16, 64
    E = 5
    qw, _ = make_experts(919, E, N, K, levels, group, seed=0)
    T = 40
    X = to_dev(wl.gaussian(wl.rng(919, 1), T, K), torch.bfloat16)
    counts = [0, 150, 0, 1, 3]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    g = wl.rng(919, 2)
    row_token = g.integers(0, T, offsets[-1]).astype(np.int32)
    row_token[7] = T + 5
    y = tq.gather_qmm(qw, X, torch.from_numpy(row_token).cuda(), torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    yg = as_f64(y)
    assert np.isnan(yg[7]).all()
    codes, scales = gpu_arrays(qw)
    Xf = as_f64(X)
    for e in range(E):
        for m in range(offsets[e], offsets[e + 1]):
            if m == 7:
                continue
            want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 0, Xf[row_token[m]])
            check_outputs(yg[m], want, bound, f"row {m}")
    # pre-rotated bf16 input gives the same rows within bf16 rounding of x'
    Xr = to_dev(ohd.rotate(Xf, 0).astype(np.float32), torch.bfloat16)
    y2 = tq.gather_qmm(qw, Xr, torch.from_numpy(row_token).cuda(), torch.from_numpy(offsets).cuda(),
                       rotated=True)
    torch.cuda.synchronize()
    ok = np.ones(offsets[-1], bool)
    ok[7] = False
    assert np.allclose(as_f64(y2)[ok], yg[ok], rtol=0, atol=2e-2 * np.abs(yg[ok]).max())


def test_gather_qmm_many_experts():
    # more experts than the schedule kernel's threads hold one by one (blocks of experts per
    # thread), most of them empty, an expert whose rows span several 128-row tiles, and a
    # column count that leaves the last 512-column tile partial
    K, N, levels, group = 256, 600, 16, 64
    E = 1500
    g = wl.rng(921, 1)
    codes = torch.from_numpy(g.integers(0, 2**31 - 1, (E, N, K // 8), dtype=np.int64).astype(np.int32)).cuda()
    scales = torch.from_numpy((g.random((E, N, K // group)) * 0.02 + 0.005).astype(np.float16)).cuda()
    qw = tq.QWeight(codes, scales, tq.signs(0, K, torch.device("cuda")), levels, group, K, N, E, 0)
    counts = np.zeros(E, np.int64)
    counts[[3, 700, 1024, 1025, 1499]] = [5, 300, 1, 17, 2]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = 50
    row_token = g.integers(0, T, offsets[-1]).astype(np.int32)
    X = to_dev(wl.gaussian(wl.rng(921, 2), T, K), torch.bfloat16)
    y = tq.gather_qmm(qw, X, torch.from_numpy(row_token).cuda(), torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    cs, ss = gpu_arrays(qw)
    Xf = as_f64(X)
    yg = as_f64(y)
    for e in np.nonzero(counts)[0]:
        a, b = offsets[e], offsets[e + 1]
        want, bound = qmv_reference(cs[e], ss[e], levels, group, K, 0, Xf[row_token[a:b]])
        check_outputs(yg[a:b], want, bound, f"expert {e}")


# output rounding of each result type, relative to the value (round to nearest)
OUT_ROUND = {torch.float32: 0.0, torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11}


@pytest.mark.parametrize("xdt", [torch.float32, torch.float16])
@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float16])
def test_gather_family_dtypes(xdt, ydt):
    # every input and output type through gather_qmv, multi_gather_qmv and gather_qmm (the
    # other tests of these three use bf16 inputs and fp32 results)
    E, N, K, levels, group = 6, 72, 1024, 16, 64
    qw, _ = make_experts(925, E, N, K, levels, group, seed=3)
    codes, scales = gpu_arrays(qw)
    g = wl.rng(925, 1)
    # gather_qmv: one input, several experts
    x = to_dev(wl.gaussian(g, 1, K)[0], xdt)
    ids = torch.tensor([5, 0, 2, 5], dtype=torch.int32, device="cuda")
    y = tq.gather_qmv(qw, ids, x, out_dtype=ydt)
    torch.cuda.synchronize()
    assert y.dtype == ydt
    xf = as_f64(x)
    for k, e in enumerate([5, 0, 2, 5]):
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 3, xf)
        check_outputs(as_f64(y[k]), want, bound + OUT_ROUND[ydt] * np.abs(want), f"gather_qmv {k}")
    # multi_gather_qmv: an input per pair
    pids = np.array([1, 4, 4, 0, 3, 1, 1], dtype=np.int32)
    X = to_dev(wl.gaussian(g, len(pids), K), xdt)
    y = tq.multi_gather_qmv(qw, torch.from_numpy(pids).cuda(), X, out_dtype=ydt)
    torch.cuda.synchronize()
    assert y.dtype == ydt
    Xf = as_f64(X)
    for k, e in enumerate(pids):
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 3, Xf[k])
        check_outputs(as_f64(y[k]), want, bound + OUT_ROUND[ydt] * np.abs(want), f"multi_gather {k}")
    # gather_qmm: rows sorted by expert
    T = 40
    row_token, _, offsets = routing_case(T, E, 2, 925)
    X = to_dev(wl.gaussian(g, T, K), xdt)
    y = tq.gather_qmm(qw, X, torch.from_numpy(row_token).cuda(), torch.from_numpy(offsets).cuda(),
                      out_dtype=ydt)
    torch.cuda.synchronize()
    assert y.dtype == ydt
    Xf = as_f64(X)
    yg = as_f64(y)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if b == a:
            continue
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 3, Xf[row_token[a:b]])
        check_outputs(yg[a:b], want, bound + OUT_ROUND[ydt] * np.abs(want), f"gather_qmm expert {e}")


def test_gather_and_multi_gather_pre_rotated_inputs():
    # inputs already rotated on the caller's side (fp32 x' = H diag(s) x / sqrt(K)): the same
    # products as the oracle's on the unrotated x, within the fp32 rounding of x'
    E, N, K, levels, group = 5, 64, 2560, 8, 64
    qw, _ = make_experts(926, E, N, K, levels, group, seed=6)
    codes, scales = gpu_arrays(qw)
    g = wl.rng(926, 1)
    x = wl.gaussian(g, 1, K)[0].astype(np.float64)
    xr = torch.from_numpy(ohd.rotate(x, 6).astype(np.float32)).cuda()
    ids = [4, 1, 1, 0]
    y = tq.gather_qmv(qw, torch.tensor(ids, dtype=torch.int32, device="cuda"), xr, rotated=True)
    torch.cuda.synchronize()
    for k, e in enumerate(ids):
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 6, x)
        check_outputs(as_f64(y[k]), want, bound + 1e-6 * np.abs(want), f"gather_qmv {k}")
    X = wl.gaussian(g, 6, K).astype(np.float64)
    Xr = torch.from_numpy(np.stack([ohd.rotate(X[i], 6) for i in range(6)]).astype(np.float32)).cuda()
    pids = np.array([2, 2, 3, 0, 4, 2], dtype=np.int32)
    y = tq.multi_gather_qmv(qw, torch.from_numpy(pids).cuda(), Xr, rotated=True)
    torch.cuda.synchronize()
    for k, e in enumerate(pids):
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 6, X[k])
        check_outputs(as_f64(y[k]), want, bound + 1e-6 * np.abs(want), f"multi_gather {k}")


@pytest.mark.parametrize("K", [4096, 1536])
def test_rotation_comes_from_the_sign_bits_alone(K):
    # the descriptor holds the sign bits and no seed: a weight encoded with seed 3 but given
    # the sign bits of seed 8 is applied with seed 8's rotation (the oracle's qmv with seed
    # 8 on the same codes), and with its own sign bits it matches seed 3
    levels, group, N = 16, 64, 64
    g = wl.rng(975, K)
    W = to_dev(wl.student_rows(g, N, K), torch.bfloat16)
    x = to_dev(wl.gaussian(g, 1, K)[0], torch.bfloat16)
    qw = tq.encode(W, levels, group, 3)
    other = tq.QWeight(qw.codes, qw.scales, tq.signs(8, K), levels, group, K, N, 1, 8)
    y_own, y_other = tq.qmv(qw, x), tq.qmv(other, x)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    for y, seed in ((y_own, 3), (y_other, 8)):
        want, bound = qmv_reference(codes[0], scales[0], levels, group, K, seed, as_f64(x))
        check_outputs(as_f64(y), want, bound, f"signs of seed {seed}")
    assert not torch.allclose(y_own, y_other)
