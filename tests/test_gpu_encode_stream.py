"""tq_encode_stream (host rows streamed through a device staging buffer) writes the same
bytes as tq_encode of the whole weight on the device: chunks of a few rows with a ragged
last chunk, one chunk exactly, pinned and pageable host memory, copies on their own stream
or on the encode stream, every weight dtype and code format."""

import ctypes

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from oracle import encode as oenc
from parity import as_f64, check_codes, check_scales, torch_to_np

pytestmark = pytest.mark.gpu


def staging_for(rows_per_chunk, K, dtype):
    row = K * torch.tensor([], dtype=dtype).element_size()
    return 2 * ((rows_per_chunk * row + 255) // 256 * 256)


@pytest.mark.parametrize("levels,group,K,E,N,dtype,pinned,chunk_rows,own_stream", [
    (16, 64, 1536, 3, 50, torch.bfloat16, True, 7, True),      # 22 chunks, last one of 3 rows
    (3, 16, 2048, 1, 33, torch.float32, False, 5, True),       # pageable host memory
    (8, 128, 4096, 2, 64, torch.float16, True, 128, True),     # one chunk, exactly full
    (4, 32, 7168, 1, 9, torch.bfloat16, True, 2, False),       # copies on the encode stream
    (16, 16, 768, 4, 17, torch.float32, True, 1, True),        # one row per chunk
])
def test_encode_stream_matches_encode(levels, group, K, E, N, dtype, pinned, chunk_rows,
                                      own_stream):
    g = wl.rng(960, levels, K)
    W = torch.from_numpy(wl.student_rows(g, E * N, K)).to(dtype).view(E, N, K)
    if pinned:
        W = W.pin_memory()
    staging = staging_for(chunk_rows, K, dtype)
    cs = None if own_stream else torch.cuda.current_stream()
    qs = tq.encode_stream(W, levels, group, seed=21, staging_bytes=staging, copy_stream=cs)
    qd = tq.encode(W.cuda(), levels, group, seed=21)
    torch.cuda.synchronize()
    assert torch.equal(qs.codes, qd.codes)
    assert torch.equal(qs.scales.view(torch.int16), qd.scales.view(torch.int16))
    assert torch.equal(qs.signs, qd.signs)


def test_encode_stream_into_existing_weight_twice():
    # out= an existing weight, then a second call with other rows into the same buffers
    # (the staging halves and events of the first call are done with by then)
    levels, group, K, N = 8, 64, 1024, 40
    g = wl.rng(961, 0)
    out = tq.encode(torch.zeros((N, K), dtype=torch.bfloat16, device="cuda"), levels, group, 3)
    for rep in range(2):
        W = torch.from_numpy(wl.student_rows(g, N, K)).to(torch.bfloat16).pin_memory()
        q = tq.encode_stream(W, levels, group, seed=3, staging_bytes=staging_for(6, K, W.dtype),
                             out=out)
        qd = tq.encode(W.cuda(), levels, group, seed=3)
        torch.cuda.synchronize()
        assert q.codes.data_ptr() == out.codes.data_ptr()
        assert torch.equal(q.codes, qd.codes), rep
        assert torch.equal(q.scales.view(torch.int16), qd.scales.view(torch.int16)), rep


@pytest.mark.parametrize("levels,group,K,dtype", [(4, 64, 7168, torch.bfloat16),
                                                  (3, 16, 768, torch.float32),
                                                  (8, 128, 4096, torch.float16)])
def test_encode_stream_matches_oracle(levels, group, K, dtype):
    # the streamed encode checked against the oracle directly (not only against tq_encode):
    # sampled rows from every chunk, the ragged last chunk included
    E, N, chunk = 3, 70, 23
    g = wl.rng(962, levels, K)
    W = torch.from_numpy(wl.student_rows(g, E * N, K)).to(dtype).view(E, N, K).pin_memory()
    q = tq.encode_stream(W, levels, group, seed=5, staging_bytes=staging_for(chunk, K, dtype))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, E * N, 11), [E * N - 1, chunk - 1, chunk]]))
    Wr = as_f64(W.view(E * N, K)[torch.from_numpy(rows)])
    ref = oenc.encode(Wr, levels, group, 5)
    check_codes(torch_to_np(q.codes).reshape(E * N, -1)[rows], ref, levels, K, "stream")
    check_scales(torch_to_np(q.scales).reshape(E * N, -1)[rows], ref, "stream")


def test_back_to_back_calls_reuse_one_staging_buffer():
    # two tq_encode_stream calls through the C ABI, one staging buffer, one copy stream, and
    # nothing between them (no host sync, no stream wait): the second call's first copies
    # must wait for the first call's last encodes, which still read the staging halves
    levels, group, K, rows = 16, 64, 2048, 96
    L = tq.lib()
    g = wl.rng(963, 0)
    Ws = [torch.from_numpy(wl.student_rows(g, rows, K)).to(torch.bfloat16).pin_memory()
          for _ in range(2)]
    nbytes = staging_for(4, K, torch.bfloat16)
    staging = torch.empty(nbytes // 8, dtype=torch.int64, device="cuda")
    wpr = tq.words_per_row(K, levels)
    outs = [(torch.empty((rows, wpr), dtype=torch.int32, device="cuda"),
             torch.empty((rows, K // group), dtype=torch.float16, device="cuda")) for _ in Ws]
    copy = torch.cuda.Stream()
    enc = torch.cuda.current_stream()
    for W, (c, s) in zip(Ws, outs):
        rc = L.tq_encode_stream(ctypes.c_void_p(W.data_ptr()), tq.BF16, rows, K, levels, group,
                                9, ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(s.data_ptr()),
                                ctypes.c_void_p(staging.data_ptr()), nbytes,
                                ctypes.c_void_p(enc.cuda_stream),
                                ctypes.c_void_p(copy.cuda_stream))
        assert rc == 0, L.tq_last_error()
    torch.cuda.synchronize()
    for W, (c, s) in zip(Ws, outs):
        ref = tq.encode(W.cuda(), levels, group, 9)
        torch.cuda.synchronize()
        assert torch.equal(c, ref.codes[0])
        assert torch.equal(s.view(torch.int16), ref.scales[0].view(torch.int16))
