"""GPU parity of tq_signs, tq_fwht and tq_encode against the oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from oracle import encode as oenc
from oracle import hadamard as ohd
from parity import as_f64, check_codes, check_scales, torch_to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def to_dev(a, dtype):
    """numpy fp32 -> torch tensor of `dtype` on the GPU (bf16 rounded to nearest even)."""
    if dtype == torch.bfloat16:
        bits = wl.f32_to_bf16_bits(a)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)


@pytest.mark.parametrize("K", [64, 512, 768, 1536, 4096, 7168, 640, 8192])
def test_signs(K):
    for seed in (0, 1, 12345):
        bits = torch_to_np(tq.signs(seed, K))
        s = ohd.signs(seed, K)
        got = np.array([(bits[i >> 5] >> (i & 31)) & 1 for i in range(K)])
        np.testing.assert_array_equal(got, (s < 0).astype(np.int64))


@pytest.mark.parametrize("K", [64, 512, 768, 1536, 2048, 4096, 7168, 640, 96, 8192, 6144, 5120])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_fwht(K, dtype):
    g = wl.rng(900, K)
    x = to_dev(wl.gaussian(g, 5, K, outliers=3), dtype)
    out = tq.fwht(x, seed=7, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = ohd.rotate(as_f64(x), 7)
    err = np.abs(as_f64(out) - want)
    tol = 1e-5 * np.linalg.norm(as_f64(x), axis=1, keepdims=True)
    assert np.all(err <= tol), float(np.max(err / tol))


CASES = [
    # (levels, group, K, rows, dtype)  -- the five workloads' shapes, fewer rows
    (16, 64, 512, 256, torch.float32),     # single layer 256x512 fp32, 4-bit g64 (all rows)
    (8, 128, 4096, 512, torch.bfloat16),   # dense 4096x4096, 3-bit g128
    (4, 64, 7168, 96, torch.bfloat16),     # MoE gate/up, 2-bit g64, K = 28 * 256
    (16, 64, 2048, 96, torch.bfloat16),    # MoE down, 4-bit g64
    (3, 16, 2048, 96, torch.bfloat16),     # ternary gate/up, g16
    (3, 16, 768, 96, torch.bfloat16),      # ternary down, K = 12 * 64
    (16, 128, 4096, 64, torch.bfloat16),   # batched gate/up, 4-bit g128
    (16, 128, 1536, 64, torch.bfloat16),   # batched down, K = 12 * 128
]


@pytest.mark.parametrize("levels,group,K,rows,dtype", CASES)
def test_encode_configs(levels, group, K, rows, dtype):
    g = wl.rng(901, levels * 1000 + group, K)
    W = to_dev(wl.student_rows(g, rows, K), dtype)
    qw = tq.encode(W, levels, group, seed=0)
    torch.cuda.synchronize()
    ref = oenc.encode(as_f64(W), levels, group, 0)
    n = check_codes(torch_to_np(qw.codes).reshape(rows, -1), ref, levels, K, f"L{levels} g{group} K{K}")
    check_scales(torch_to_np(qw.scales).reshape(rows, -1), ref)
    if levels == 16 and K == 512:
        assert n == 0  # the small layer must be bit-exact


DTYPES = [torch.float16, torch.bfloat16, torch.float32]


@pytest.mark.parametrize("levels", [3, 4, 8, 16])
@pytest.mark.parametrize("group", [16, 32, 64, 128])
@pytest.mark.parametrize("K", [1536, 2048, 256, 4096, 128])
def test_encode_all_formats(levels, group, K):
    # K = 12 * 128 takes the 12-point factor; the powers of two take the register kernel
    # in each of its layouts (one exchange for K <= 512, two for K >= 1024); 41 rows leave
    # a partial batch of rows
    if group > K:
        pytest.skip("group larger than the row")
    g = wl.rng(902, levels * 1000 + group, K)
    dtype = DTYPES[(levels + group // 16 + K // 128) % 3]
    W = to_dev(wl.student_rows(g, 41, K), dtype)
    qw = tq.encode(W, levels, group, seed=3)
    torch.cuda.synchronize()
    ref = oenc.encode(as_f64(W), levels, group, 3)
    check_codes(torch_to_np(qw.codes).reshape(41, -1), ref, levels, K)
    check_scales(torch_to_np(qw.scales).reshape(41, -1), ref)


@pytest.mark.parametrize("K", [64, 128, 256, 512, 1024, 2048, 4096])
@pytest.mark.parametrize("dtype", DTYPES)
def test_encode_power_of_two_rows(K, dtype):
    # every power-of-two row length of the register kernel, every input dtype, with edge
    # rows (zero, constant, huge and tiny magnitudes) among ordinary ones
    levels, group = 16, 64 if K >= 64 else K
    g = wl.rng(908, K)
    W = wl.student_rows(g, 70, K)
    W[3] = 0.0
    W[5, :] = 1.0
    W[7] *= 1e2 if dtype == torch.float16 else 1e6  # fp16 holds at most 65504
    W[9] *= 1e-3 if dtype == torch.float16 else 1e-6
    Wd = to_dev(W, dtype)
    qw = tq.encode(Wd, levels, group, seed=17)
    torch.cuda.synchronize()
    ref = oenc.encode(as_f64(Wd), levels, group, 17)
    check_codes(torch_to_np(qw.codes).reshape(70, -1), ref, levels, K)
    check_scales(torch_to_np(qw.scales).reshape(70, -1), ref)


@pytest.mark.parametrize("m", [12, 20, 28])
@pytest.mark.parametrize("P", [32, 64, 128, 256])
def test_encode_m_layouts(m, P):
    # every layout of the register kernel for rows of m * P (P = 32: no middle exchange;
    # 64 .. 256: one, with 1 .. 3 stages), every input dtype and bit or trit format across the
    # cases (256 levels are for power-of-two rows only),
    # edge rows among ordinary ones, and a row count that leaves a partial batch
    K = m * P
    levels = [3, 4, 8, 16][(m + P // 32) % 4]
    group = [16, 32, 64, 128][(m // 4 + P // 64) % 4]
    dtype = DTYPES[(m + P) % 3]
    rows = 16384 // K * 2 + 3
    g = wl.rng(911, m, P)
    W = wl.student_rows(g, rows, K)
    W[1] = 0.0
    W[2, :] = 1.0
    W[4] *= 1e2 if dtype == torch.float16 else 1e5
    Wd = to_dev(W, dtype)
    qw = tq.encode(Wd, levels, group, seed=23)
    torch.cuda.synchronize()
    ref = oenc.encode(as_f64(Wd), levels, group, 23)
    check_codes(torch_to_np(qw.codes).reshape(rows, -1), ref, levels, K, f"m{m} P{P} L{levels} g{group}")
    check_scales(torch_to_np(qw.scales).reshape(rows, -1), ref)


def test_encode_edge_rows():
    # zero rows, a row with one zero group, huge and tiny magnitudes (fp16 scale saturation
    # and subnormal scales), and a constant row
    K, levels, group = 640, 8, 32  # K = 20 * 32: the 20-point factor
    g = wl.rng(903, 0)
    W = wl.student_rows(g, 8, K).astype(np.float32)
    W[0] = 0.0
    W[1, :] = 1.0
    W[2] *= 1e6
    W[3] *= 1e-6
    W[4, :32] = 0.0  # rotation spreads this; the row is still non-zero
    Wd = to_dev(W, torch.float32)
    qw = tq.encode(Wd, levels, group, seed=5)
    torch.cuda.synchronize()
    ref = oenc.encode(W.astype(np.float64), levels, group, 5)
    check_codes(torch_to_np(qw.codes).reshape(8, -1), ref, levels, K)
    check_scales(torch_to_np(qw.scales).reshape(8, -1), ref)
    sc = torch_to_np(qw.scales).reshape(8, -1)
    assert np.all(sc[0] == 0)
    assert np.all(sc[2] == 0x7BFF)  # saturated


def test_encode_chunk_invariance_and_determinism():
    K, levels, group = 2048, 16, 64
    g = wl.rng(904, 0)
    W = to_dev(wl.student_rows(g, 300, K), torch.bfloat16)
    a = tq.encode(W, levels, group, seed=9)
    b = tq.encode(W, levels, group, seed=9)
    parts = [tq.encode(W[i:i + 77], levels, group, seed=9) for i in range(0, 300, 77)]
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes) and torch.equal(a.scales.view(torch.int16), b.scales.view(torch.int16))
    cat_c = torch.cat([p.codes for p in parts], dim=1)
    cat_s = torch.cat([p.scales for p in parts], dim=1)
    assert torch.equal(a.codes, cat_c)
    assert torch.equal(a.scales.view(torch.int16), cat_s.view(torch.int16))


def test_encode_expert_stack_shape():
    K, levels, group = 768, 3, 16
    g = wl.rng(905, 0)
    W = to_dev(wl.student_rows(g, 3 * 50, K), torch.bfloat16).view(3, 50, K)
    qw = tq.encode(W, levels, group, seed=1)
    torch.cuda.synchronize()
    assert qw.codes.shape == (3, 50, 39) and qw.scales.shape == (3, 50, 48)
    ref = oenc.encode(as_f64(W.reshape(150, K)), levels, group, 1)
    check_codes(torch_to_np(qw.codes).reshape(150, -1), ref, levels, K)


@pytest.mark.parametrize("levels,group,K", [(4, 64, 7168), (3, 16, 768), (16, 64, 1536),
                                            (8, 128, 4096)])
def test_encode_many_rows_in_one_call(levels, group, K):
    # 3 * 4096 + 17 rows in one tq_encode call, the way expert stacks are encoded (16
    # experts at a time); sampled rows, among them the first and last rows of each block of
    # 4096 and the ragged tail, checked against the oracle's encode of the same bytes
    rows = 3 * 4096 + 17
    gen = wl.torch_generator(torch.device(DEV), 907, levels, K)
    W = wl.torch_student_rows(gen, rows, K, DEV, torch.bfloat16)
    qw = tq.encode(W, levels, group, seed=2)
    torch.cuda.synchronize()
    g = wl.rng(907, levels, K)
    edges = [0, 1, 4095, 4096, 4097, 8191, 8192, 12287, 12288, rows - 2, rows - 1]
    sample = np.unique(np.concatenate([edges, g.choice(rows, 40, replace=False)]))
    idx = torch.from_numpy(sample).to(DEV)
    ref = oenc.encode(as_f64(W[idx]), levels, group, 2)
    codes = torch_to_np(qw.codes[0][idx]).reshape(len(sample), -1)
    scales = torch_to_np(qw.scales[0][idx]).reshape(len(sample), -1)
    check_codes(codes, ref, levels, K, f"L{levels} K{K} {rows} rows")
    check_scales(scales, ref, f"L{levels} K{K} {rows} rows")
