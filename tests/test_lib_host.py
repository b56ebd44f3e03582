"""Host-side checks of libtq.so that need no GPU.

* The shared library loads and exports every function declared in include/tq.h, and the
  binding declares a signature for each of them (no kernel is launched here).
* The library's Lloyd-Max codebook, computed by its own C++ Lloyd iteration, equals the
  oracle's fp64 codebook rounded once to binary32, bit for bit (centroids and thresholds).
* Argument validation rejects bad shapes, levels, groups, dtypes, null pointers,
  misalignment and short workspaces with the documented status, before any launch.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import rotation_lloyd_max_amd as tq
from oracle import codebook as ocb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tq.LIB_PATH),
                                reason="libtq.so not built (run __graft_entry__.build())")

ERR_ARG, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE = -1, -2, -3, -4


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) == 24, names
    handle = ctypes.CDLL(tq.LIB_PATH)
    for n in names:
        assert hasattr(handle, n), n
    assert sorted(s[0] for s in tq.SIGNATURES) == names


@pytest.mark.parametrize("L", [3, 4, 8, 16, 256])
def test_codebook_matches_oracle_bitwise(L):
    c, t = tq.codebook(L)
    oc, ot, _, _ = ocb.lloyd_max(L)
    np.testing.assert_array_equal(c.view(np.uint32), oc.astype(np.float32).view(np.uint32))
    np.testing.assert_array_equal(t.view(np.uint32), ot.astype(np.float32).view(np.uint32))


def test_codebook_rejects_other_levels():
    for L in (0, 1, 2, 5, 32, 255):
        with pytest.raises(tq.TqError) as e:
            tq.codebook(L)
        assert e.value.status == ERR_UNSUPPORTED


def test_words_per_row():
    assert tq.words_per_row(4096, 8) == 384
    assert tq.words_per_row(7168, 4) == 448
    assert tq.words_per_row(2048, 3) == 103
    assert tq.words_per_row(512, 16) == 64
    assert tq.words_per_row(512, 5) == 0


def desc(**kw):
    d = dict(codes=16, scales=16, signs=16, n_levels=16, group=64, K=512, N=4, E=1)
    d.update(kw)
    return tq._QWeight(d["codes"], d["scales"], d["signs"], d["n_levels"], d["group"], d["K"],
                       d["N"], d["E"])


def test_descriptor_holds_one_rotation():
    # tq_qweight carries the sign bits and no seed: the header's struct and the binding's
    # mirror of it list the same fields, in the same order, and "seed" is not one of them
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} tq_qweight;", text, flags=re.S).group(1)
    fields = re.findall(r"\b(\w+)\s*[;,]", body)
    assert fields == [f[0] for f in tq._QWeight._fields_], fields
    assert "seed" not in fields and "signs" in fields
    assert ctypes.sizeof(tq._QWeight) == 3 * 8 + 2 * 4 + 3 * 8
    # without sign bits there is no rotation: rejected before any launch
    assert qmv_status(desc(signs=0)) == ERR_ARG
    assert b"signs" in tq.lib().tq_last_error()


def qmv_status(d, x=16, xdt=0, y=16, ydt=0):
    return tq.lib().tq_qmv(ctypes.byref(d) if d is not None else None, x, xdt, y, ydt, 0, None,
                           0, None)


def test_validation_statuses():
    L = tq.lib()
    assert qmv_status(None) == ERR_ARG
    assert qmv_status(desc(n_levels=5)) == ERR_UNSUPPORTED
    assert qmv_status(desc(group=8)) == ERR_UNSUPPORTED
    assert qmv_status(desc(K=4864)) == ERR_UNSUPPORTED     # 4864 = 19 * 256: no Hadamard
    # ...but a pre-rotated input needs none (N = 0: accepted, and nothing is launched)
    assert tq.lib().tq_qmv(ctypes.byref(desc(K=4864, signs=0, N=0)), 16, 0, 16, 0, 1, None, 0,
                           None) == 0
    assert tq.lib().tq_qmv(ctypes.byref(desc(K=4864, signs=0, N=0)), 16, 0, 16, 0, 0, None, 0,
                           None) == ERR_UNSUPPORTED
    assert qmv_status(desc(K=16384)) == ERR_UNSUPPORTED    # above the size limit
    assert qmv_status(desc(K=96, group=64)) == ERR_UNSUPPORTED  # group does not divide K
    assert qmv_status(desc(codes=0)) == ERR_ARG
    assert qmv_status(desc(codes=8)) == ERR_ALIGN
    assert qmv_status(desc(E=2)) == ERR_ARG                # dense qmv needs E = 1
    assert qmv_status(desc(), xdt=7) == ERR_ARG
    assert qmv_status(desc(), x=0) == ERR_ARG
    assert qmv_status(desc(), x=18, xdt=0) == ERR_ALIGN
    assert qmv_status(desc(), x=20, xdt=0) == ERR_ALIGN  # x needs 16-byte alignment
    assert b"group" in L.tq_last_error() or L.tq_last_error()
    # multi_gather: short workspace
    d = desc(E=4)
    need = L.tq_workspace_bytes(3, ctypes.byref(d), 10, 0)
    assert 0 < need < 1 << 20
    assert L.tq_multi_gather_qmv(ctypes.byref(d), 16, 10, 16, 0, 16, 0, 0, 256, need - 1,
                                 None) == ERR_WORKSPACE
    # gather_qmm: workspace alignment and size
    need = L.tq_workspace_bytes(4, ctypes.byref(d), 100, 50)
    assert need >= 50 * 512 * 2
    assert L.tq_gather_qmm(ctypes.byref(d), 16, 1, 50, 16, 16, 100, 16, 0, 0, 256, 10,
                           None) == ERR_WORKSPACE
    assert L.tq_gather_qmm(ctypes.byref(d), 16, 1, 50, 16, 16, 100, 16, 0, 0, 128, need,
                           None) == ERR_ALIGN
    # dequant: more blocks than experts without ids, misaligned output, bad dtype, bad n
    assert L.tq_dequant(ctypes.byref(d), None, 5, 256, 1, None) == ERR_ARG
    assert L.tq_dequant(ctypes.byref(d), None, 2, 258, 1, None) == ERR_ALIGN
    assert L.tq_dequant(ctypes.byref(d), 16, 2, 256, 7, None) == ERR_ARG
    assert L.tq_dequant(ctypes.byref(d), 16, 70000, 256, 1, None) == ERR_ARG
    assert L.tq_dequant(ctypes.byref(d), 18, 2, 256, 1, None) == ERR_ALIGN
    # encode / fwht / signs
    assert L.tq_encode(16, 0, 4, 500, 16, 64, 0, 16, 16, None) == ERR_UNSUPPORTED
    assert L.tq_encode(0, 0, 4, 512, 16, 64, 0, 16, 16, None) == ERR_ARG
    assert L.tq_encode(16, 0, -1, 512, 16, 64, 0, 16, 16, None) == ERR_ARG
    assert L.tq_fwht(16, 0, 2, 100, 0, 16, 0, None) == ERR_UNSUPPORTED
    assert L.tq_signs(0, 0, 16, None) == ERR_ARG
    # encode_stream: checked before any copy or launch (no GPU needed): unsupported K, NULL
    # host rows or staging, misaligned staging, staging under two rows (K 512 fp32 = 2 KB a
    # row: 4 KB is the least), and nothing to do for zero rows
    es = L.tq_encode_stream
    assert es(16, 0, 4, 500, 16, 64, 0, 16, 16, 256, 1 << 20, None, None) == ERR_UNSUPPORTED
    assert es(0, 0, 4, 512, 16, 64, 0, 16, 16, 256, 1 << 20, None, None) == ERR_ARG
    assert es(16, 0, 4, 512, 16, 64, 0, 16, 16, 0, 1 << 20, None, None) == ERR_ARG
    assert es(16, 0, 4, 512, 16, 64, 0, 16, 16, 128, 1 << 20, None, None) == ERR_ALIGN
    assert es(16, 0, 4, 512, 16, 64, 0, 16, 16, 256, 4095, None, None) == ERR_ARG
    assert b"fewer than two rows" in L.tq_last_error()
    assert es(16, 3, 4, 512, 16, 64, 0, 16, 16, 256, 1 << 20, None, None) == ERR_ARG
    assert es(16, 0, 0, 512, 16, 64, 0, 16, 16, 256, 0, None, None) == 0
    # the allocation-free multi_gather refuses a call whose workspace exceeds its fixed 8 MiB
    # (4000 pairs of K = 2048), before touching the device
    d2 = desc(E=4, K=2048, n_levels=3, group=16)
    assert L.tq_multi_gather_qmv_static(ctypes.byref(d2), 16, 4000, 16, 1, 16, 0, 0,
                                        None) == ERR_WORKSPACE
    assert b"8388608" in L.tq_last_error()
    assert L.tq_multi_gather_qmv_static(ctypes.byref(d2), None, 4, 16, 1, 16, 0, 0,
                                        None) == ERR_ARG
    # dense rotation: shapes, pointers, workspace
    assert L.tq_rotate_dense(16, 0, 2, 100, 16, 16, 0, None) == ERR_UNSUPPORTED
    assert L.tq_rotate_dense(16, 0, 2, 4864, 0, 16, 0, None) == ERR_ARG
    assert L.tq_rotate_dense(16, 0, 2, 4864, 18, 16, 0, None) == ERR_ALIGN
    assert L.tq_rotate_dense(0, 0, 0, 4864, 0, 0, 0, None) == 0
    assert L.tq_encode_dense(16, 1, 4, 4864, 16, 8, 128, 16, 16, 16, 4864 * 8 - 1,
                             None) == ERR_WORKSPACE
    assert L.tq_encode_dense(16, 1, 4, 4864, 16, 8, 100, 16, 16, 16, 1 << 20,
                             None) == ERR_UNSUPPORTED
    assert L.tq_workspace_bytes(5, ctypes.byref(desc(K=4864, signs=0)), 10, 0) == 10 * 4864 * 8
    # KV fetch: formats and lengths outside its set are refused; 256 levels only there
    assert L.tq_kv_fetch(ctypes.byref(desc(n_levels=3, group=16)), 256, 1, None) == ERR_UNSUPPORTED
    assert L.tq_kv_fetch(ctypes.byref(desc(K=4096)), 256, 1, None) == ERR_UNSUPPORTED
    assert L.tq_kv_fetch(ctypes.byref(desc(K=768, group=64)), 256, 1, None) == ERR_UNSUPPORTED
    assert L.tq_kv_fetch(ctypes.byref(desc(n_levels=256)), 258, 1, None) == ERR_ALIGN
    assert L.tq_kv_fetch(ctypes.byref(desc(n_levels=256)), 256, 9, None) == ERR_ARG
    assert qmv_status(desc(n_levels=256)) == ERR_UNSUPPORTED
    assert L.tq_encode(16, 1, 4, 768, 256, 64, 0, 16, 16, None) == ERR_UNSUPPORTED
    assert L.tq_encode(18, 1, 4, 512, 256, 64, 0, 16, 16, None) == ERR_ALIGN
    assert L.tq_words_per_row(128, 256) == 32
    # expert cache: sizes, set-up checks, and fetches refused before anything is enqueued
    assert L.tq_expert_cache_bytes(0, 10) == ctypes.c_size_t(-1).value
    nb = L.tq_expert_cache_bytes(4, 10)
    st = np.zeros(nb // 8 + 1, dtype=np.uint64)
    assert L.tq_expert_cache_init(st.ctypes.data, nb - 1, 4, 10) == ERR_ARG
    assert L.tq_expert_cache_init(st.ctypes.data + 4, nb, 4, 10) == ERR_ALIGN
    assert L.tq_expert_cache_init(st.ctypes.data, nb, 4, 10) == 0
    hostw, pool = desc(E=10), desc(E=4)
    fetch = lambda ids, p=pool: L.tq_expert_cache_fetch(
        st.ctypes.data, ctypes.byref(hostw), ctypes.byref(p),
        np.asarray(ids, dtype=np.int32).ctypes.data, len(ids), 256, None, None, None, None)
    assert fetch([0, 10]) == ERR_ARG                      # id outside [0, E)
    assert fetch([0, 1, 2, 3, 4]) == ERR_ARG              # five distinct experts, four slots
    assert fetch([1], desc(E=5)) == ERR_ARG               # pool is not the cache's slots
    assert fetch([1], desc(E=4, group=32)) == ERR_ARG     # pool of another format
    h, m = ctypes.c_int64(7), ctypes.c_int64(7)
    assert L.tq_expert_cache_stats(st.ctypes.data, ctypes.byref(h), ctypes.byref(m)) == 0
    assert (h.value, m.value) == (0, 0)                   # refused fetches left no trace
    assert L.tq_expert_cache_stats(np.zeros(8, dtype=np.uint64).ctypes.data, None, None) == ERR_ARG
    # workspace query with a bad descriptor
    assert L.tq_workspace_bytes(3, None, 1, 0) == ctypes.c_size_t(-1).value
    assert L.tq_workspace_bytes(9, ctypes.byref(desc()), 1, 0) == ctypes.c_size_t(-1).value


def test_gather_qmv_pair_validation():
    # the two weights must match in format and shape and share one signs array; every
    # rejection happens before a launch
    L = tq.lib()

    def pair(d1, d2, n=4, ids=16, flags=0):
        return L.tq_gather_qmv_pair(ctypes.byref(d1), ctypes.byref(d2), ids, n, 16, 1, 16, 0,
                                    flags, None)

    a = desc(E=3)
    assert pair(a, desc(E=3, n_levels=8)) == ERR_ARG
    assert pair(a, desc(E=3, group=128)) == ERR_ARG
    assert pair(a, desc(E=3, N=8)) == ERR_ARG
    assert pair(a, desc(E=4)) == ERR_ARG
    assert pair(a, desc(E=3, K=1024)) == ERR_ARG
    assert pair(a, desc(E=3, signs=32)) == ERR_ARG       # a second rotation
    assert pair(a, desc(E=3), n=65536) == ERR_ARG        # past the grid's y limit
    assert pair(a, desc(E=3), n=-1) == ERR_ARG
    assert pair(a, desc(E=3), ids=0) == ERR_ARG
    assert pair(a, desc(E=3), ids=18) == ERR_ALIGN
    assert pair(a, desc(E=3, codes=8)) == ERR_ALIGN
    assert L.tq_gather_qmv_pair(None, ctypes.byref(a), 16, 4, 16, 1, 16, 0, 0, None) == ERR_ARG
    # zero ids: nothing to do; a pre-rotated input reads no signs, so they need not match
    assert pair(a, desc(E=3), n=0, ids=0) == 0
    assert pair(desc(E=3, N=0, signs=0), desc(E=3, N=0, signs=16), n=4, flags=1) == 0


def test_multi_gather_qmv_pair_validation():
    L = tq.lib()
    a = desc(E=4)
    need = L.tq_workspace_bytes(3, ctypes.byref(a), 10, 0)

    def pair(d1, d2, P=10, ids=16, ws=256, nbytes=need, flags=0):
        return L.tq_multi_gather_qmv_pair(ctypes.byref(d1), ctypes.byref(d2), ids, P, 16, 1, 16,
                                          0, flags, ws, nbytes, None)

    assert pair(a, desc(E=4, n_levels=3, group=16)) == ERR_ARG
    assert pair(a, desc(E=4, N=8)) == ERR_ARG
    assert pair(a, desc(E=5)) == ERR_ARG
    assert pair(a, desc(E=4, signs=32)) == ERR_ARG
    assert pair(a, desc(E=4), P=-1) == ERR_ARG
    assert pair(a, desc(E=4), ids=0) == ERR_ARG
    assert pair(a, desc(E=4), ids=18) == ERR_ALIGN
    assert pair(a, desc(E=4), nbytes=need - 1) == ERR_WORKSPACE
    assert pair(a, desc(E=4), ws=0) == ERR_WORKSPACE
    assert pair(a, desc(E=4), ws=264) == ERR_ALIGN
    assert pair(a, desc(E=4), P=0, ids=0, ws=0, nbytes=0) == 0
    assert L.tq_multi_gather_qmv_pair(None, ctypes.byref(a), 16, 10, 16, 1, 16, 0, 0, 256, need,
                                      None) == ERR_ARG


def test_gather_qmm_pair_validation():
    L = tq.lib()
    a = desc(E=4)
    need = L.tq_workspace_bytes(4, ctypes.byref(a), 100, 50)

    def pair(d1, d2, M=100, rt=16, off=16, ws=256, nbytes=need, flags=0):
        return L.tq_gather_qmm_pair(ctypes.byref(d1), ctypes.byref(d2), 16, 1, 50, rt, off, M,
                                    16, 0, flags, ws, nbytes, None)

    assert pair(a, desc(E=4, group=128)) == ERR_ARG
    assert pair(a, desc(E=4, N=8)) == ERR_ARG
    assert pair(a, desc(E=3)) == ERR_ARG
    assert pair(a, desc(E=4, signs=32)) == ERR_ARG
    assert pair(a, desc(E=4), M=1 << 30) == ERR_ARG
    assert pair(a, desc(E=4), rt=0) == ERR_ARG
    assert pair(a, desc(E=4), off=18) == ERR_ALIGN
    assert pair(a, desc(E=4), nbytes=need - 1) == ERR_WORKSPACE
    assert pair(a, desc(E=4), ws=272) == ERR_ALIGN
    assert pair(a, desc(E=4), M=0, rt=0, off=0, ws=0, nbytes=0) == 0


def test_output_buffers_are_checked():
    # an out= buffer must hold exactly the elements a call writes, contiguously, on the
    # call's device: the library writes through its pointer
    import torch
    cpu = torch.device("cpu")
    assert tuple(tq._out(None, 7, torch.float32, cpu).shape) == (7,)
    o = torch.empty(4, 6)
    assert tq._out(o, (4, 6), torch.float32, cpu) is o
    assert tq._out(o.view(24), (4, 6), torch.float32, cpu).numel() == 24
    for bad in (torch.empty(4, 5), torch.empty(6, 4).t(), torch.empty(4, 12)[:, ::2]):
        with pytest.raises(ValueError):
            tq._out(bad, (4, 6), torch.float32, cpu)


def test_empty_calls_are_no_ops():
    L = tq.lib()
    # zero rows / zero ids / zero pairs return OK without touching the device
    assert L.tq_encode(0, 0, 0, 512, 16, 64, 0, 0, 0, None) == 0
    assert L.tq_fwht(0, 0, 0, 512, 0, 0, 0, None) == 0
    d = desc(N=0, codes=0, scales=0, signs=0)
    assert qmv_status(d, x=0, y=0) == 0
    d = desc(E=3)
    assert L.tq_gather_qmv(ctypes.byref(d), None, 0, 0, 1, 0, 0, 0, None, 0, None) == 0
    assert L.tq_multi_gather_qmv(ctypes.byref(d), None, 0, 0, 1, 0, 0, 0, None, 0, None) == 0
    assert L.tq_gather_qmm(ctypes.byref(d), 0, 1, 0, None, None, 0, 0, 0, 0, None, 0, None) == 0
    assert L.tq_dequant(ctypes.byref(d), None, 0, None, 1, None) == 0
