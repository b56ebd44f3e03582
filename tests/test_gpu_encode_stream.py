"""tq_encode_stream (host rows streamed through a device staging buffer) writes the same
bytes as tq_encode of the whole weight on the device: chunks of a few rows with a ragged
last chunk, one chunk exactly, pinned and pageable host memory, copies on their own stream
or on the encode stream, every weight dtype and code format."""

import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl

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
