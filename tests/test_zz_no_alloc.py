"""tq_multi_gather_qmv_static (the allocation-free variant of tq_multi_gather_qmv, whose
workspace is a fixed per-GPU array in the library) against tq_multi_gather_qmv, through the
C ABI: two calls in a row on the same GPU, the second with fewer pairs and a shorter K, each
bit-identical to the workspace entry point's result and within the oracle's bound."""

import ctypes

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from parity import as_f64, check_outputs, qmv_reference, torch_to_np
from test_gpu_encode import to_dev

pytestmark = pytest.mark.gpu


def call_static(qw, ids, X):
    L = tq.lib()
    y = torch.empty((ids.numel(), qw.N), dtype=torch.float32, device="cuda")
    d = qw.desc()
    rc = L.tq_multi_gather_qmv_static(ctypes.byref(d), ctypes.c_void_p(ids.data_ptr()),
                                      ids.numel(), ctypes.c_void_p(X.data_ptr()), tq.BF16,
                                      ctypes.c_void_p(y.data_ptr()), tq.F32, 0,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, L.tq_last_error()
    return y


def test_static_workspace_matches_workspace_entry_point_twice():
    # the ternary prefill shapes: gate (K 2048) with 512 pairs, then down (K 768) with 96
    cases = [(3, 16, 2048, 768, 16, 512), (3, 16, 768, 2048, 16, 96)]
    for levels, group, K, N, E, P in cases:
        g = wl.rng(980, K)
        W = to_dev(wl.student_rows(g, E * N, K), torch.bfloat16).view(E, N, K)
        qw = tq.encode(W, levels, group, 1)
        ids = torch.from_numpy(g.integers(0, E, P).astype(np.int32)).cuda()
        X = to_dev(wl.gaussian(g, P, K), torch.bfloat16)
        y_static = call_static(qw, ids, X)
        y_ws = tq.multi_gather_qmv(qw, ids, X)
        torch.cuda.synchronize()
        assert torch.equal(y_static, y_ws), f"K {K} P {P}"
        codes = torch_to_np(qw.codes).reshape(E, N, -1)
        scales = torch_to_np(qw.scales).reshape(E, N, -1)
        yg, Xf, ids_np = as_f64(y_static), as_f64(X), ids.cpu().numpy()
        for p_ in range(0, P, max(1, P // 12)):
            e = ids_np[p_]
            want, bound = qmv_reference(codes[e], scales[e], levels, group, K, 1, Xf[p_])
            check_outputs(yg[p_], want, bound, f"K {K} pair {p_}")


def test_static_workspace_rejects_calls_above_its_size():
    # 4000 pairs of K = 2048 need about 16 MB of workspace: refused before any launch
    levels, group, K, N, E = 3, 16, 2048, 64, 2
    qw = tq.encode(torch.zeros((E, N, K), dtype=torch.bfloat16, device="cuda"), levels, group, 1)
    ids = torch.zeros(4000, dtype=torch.int32, device="cuda")
    X = torch.zeros((4000, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tq.TqError) as e:
        tq.multi_gather_qmv_static(qw, ids, X)
    assert e.value.status == -4 and "8388608" in str(e.value)
