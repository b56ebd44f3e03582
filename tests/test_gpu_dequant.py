"""GPU parity of tq_dequant (decoded weights in the rotated basis) against the oracle's
dequantization of the same codes, and its use as "dequantize, then a regular matrix
multiply" next to the fused kernels."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from oracle import encode as oenc
from parity import as_f64, check_outputs, qmv_reference
from test_gpu_encode import to_dev
from test_gpu_qmv import gpu_arrays

pytestmark = pytest.mark.gpu

# significant bits kept by each output type; the fp32 path also rounds the centroid to fp32
MANT = {torch.float32: 22, torch.bfloat16: 7, torch.float16: 10}


def check_dequant(got, want, odt, tag):
    """Each value within one unit in the last place of the output type of the fp64 value."""
    g, w = as_f64(got), np.asarray(want, dtype=np.float64)
    tol = np.abs(w) * 2.0 ** -MANT[odt] + (2.0 ** -24 if odt == torch.float16 else 0.0)
    bad = np.abs(g - w) > tol
    assert not bad.any(), f"{tag}: {bad.sum()} values off, first at {np.argwhere(bad)[0]}: " \
                          f"got {g[bad][0]!r} want {w[bad][0]!r}"


def stack(cfg, E, N, K, levels, group, seed):
    W = torch.stack([to_dev(wl.student_rows(wl.rng(cfg, 30, e), N, K), torch.bfloat16)
                     for e in range(E)])
    qw = tq.encode(W, levels, group, seed)
    torch.cuda.synchronize()
    return qw


@pytest.mark.parametrize("levels,group,K,N", [(3, 16, 768, 40), (3, 32, 2048, 24),
                                              (4, 64, 7168, 16), (8, 128, 4096, 33),
                                              (16, 16, 1536, 50), (16, 128, 640, 20),
                                              (8, 32, 96, 7)])
@pytest.mark.parametrize("odt", [torch.float32, torch.bfloat16, torch.float16])
def test_dequant_all_experts(levels, group, K, N, odt):
    # every code format, groups of 16 to 128, K with a partial last trit word (768, 2048,
    # 7168), odd row counts, all three output types
    E = 3
    qw = stack(930, E, N, K, levels, group, seed=8)
    out = tq.dequant(qw, out_dtype=odt)
    torch.cuda.synchronize()
    assert out.shape == (E, N, K) and out.dtype == odt
    codes, scales = gpu_arrays(qw)
    for e in range(E):
        want = oenc.dequant(codes[e], scales[e], levels, group, K)
        check_dequant(out[e], want, odt, f"L{levels} g{group} K{K} expert {e} {odt}")


def test_dequant_ids_and_bad_ids():
    # a subset in any order, repeats, and ids outside [0, E) (blocks of NaN)
    E, N, K, levels, group = 5, 24, 512, 16, 64
    qw = stack(931, E, N, K, levels, group, seed=2)
    ids_np = np.array([4, 0, 4, E, -3, 2], dtype=np.int32)
    out = tq.dequant(qw, torch.from_numpy(ids_np).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    for k, e in enumerate(ids_np):
        if 0 <= e < E:
            check_dequant(out[k], oenc.dequant(codes[e], scales[e], levels, group, K),
                          torch.float32, f"slot {k} expert {e}")
        else:
            assert torch.isnan(out[k]).all(), k


def test_dequant_then_matmul_matches_fused_qmv():
    # "dequantize, then a regular matrix multiply": out[e] times the rotated input equals
    # the fused gather_qmv of the same experts, and the oracle's product
    E, N, K, levels, group = 4, 96, 2048, 8, 64
    qw = stack(932, E, N, K, levels, group, seed=9)
    x = to_dev(wl.gaussian(wl.rng(932, 1), 1, K)[0], torch.float32)
    W = tq.dequant(qw, out_dtype=torch.float32)
    xr = tq.fwht(x.view(1, K), qw.seed, out_dtype=torch.float32).view(K)
    y_mm = torch.matmul(W, xr)                                   # [E][N]
    ids = torch.arange(E, dtype=torch.int32, device="cuda")
    y_fused = tq.gather_qmv(qw, ids, x)
    torch.cuda.synchronize()
    codes, scales = gpu_arrays(qw)
    xf = as_f64(x)
    for e in range(E):
        want, bound = qmv_reference(codes[e], scales[e], levels, group, K, qw.seed, xf)
        check_outputs(as_f64(y_mm[e]), want, bound, f"dequant+matmul expert {e}")
        check_outputs(as_f64(y_fused[e]), want, bound, f"gather_qmv expert {e}")


def test_dequant_argument_errors():
    # rejected on the host before any launch: more blocks than experts without ids, and an
    # output that is not 16-byte aligned
    import ctypes
    qw = stack(933, 2, 8, 256, 4, 32, seed=1)
    out = torch.empty((3 * 8 * 256 + 8,), dtype=torch.bfloat16, device="cuda")
    d = qw.desc()
    L = tq.lib()
    st = tq._stream()
    assert L.tq_dequant(ctypes.byref(d), None, 3, ctypes.c_void_p(out.data_ptr()), 1, st) == -1
    assert L.tq_dequant(ctypes.byref(d), None, 2, ctypes.c_void_p(out.data_ptr() + 2), 1, st) == -3
    assert L.tq_dequant(ctypes.byref(d), None, 2, ctypes.c_void_p(out.data_ptr()), 1, st) == 0
    torch.cuda.synchronize()
