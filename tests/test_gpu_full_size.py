"""GPU parity at the full sizes of the MoE workloads, on sampled outputs, through the C ABI
and in the launch configuration bench.py times: full expert stacks encoded on the GPU, the
same routing generators, the whole batch in one call. The oracle recomputes sampled output
rows one by one from the GPU's own codes (encode parity is tested on its own)."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from parity import as_f64, check_outputs, qmv_reference, torch_to_np

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")


def encode_stack(cfg, pr, chunk=16):
    """The expert stack of projection pr, its bf16 weights drawn on the GPU chunk by chunk."""
    E, N, K = cfg.E, pr.N, pr.K
    codes = torch.empty((E, N, tq.words_per_row(K, pr.levels)), dtype=torch.int32, device=DEV)
    scales = torch.empty((E, N, K // pr.group), dtype=torch.float16, device=DEV)
    sg = tq.signs(pr.seed, K, DEV)
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        g = wl.torch_generator(DEV, cfg.cid, wl.PROJ_TENSOR[pr.name], e0)
        W = wl.torch_student_rows(g, (e1 - e0) * N, K, DEV, torch.bfloat16).view(e1 - e0, N, K)
        tq.encode(W, pr.levels, pr.group, pr.seed,
                  out=tq.QWeight(codes[e0:e1], scales[e0:e1], sg, pr.levels, pr.group, K, N, e1 - e0, pr.seed))
        del W
    torch.cuda.synchronize()
    return tq.QWeight(codes, scales, sg, pr.levels, pr.group, K, N, E, pr.seed)


def sampled_check(qw, e, rows, x_rows, y_rows, tag):
    """Oracle rows `rows` of expert e against inputs x_rows ([n][K] fp64) vs y_rows ([n][rows])."""
    codes = torch_to_np(qw.codes[e, rows]).reshape(len(rows), -1)
    scales = torch_to_np(qw.scales[e, rows]).reshape(len(rows), -1)
    want, bound = qmv_reference(codes, scales, qw.levels, qw.group, qw.K, qw.seed, x_rows)
    return check_outputs(y_rows, want, bound, tag)


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_moe_decode_gather_qmv_full_size(proj):
    # 384 experts, hidden 7168, intermediate 2048; gate 2-bit g64, down 4-bit g64; one token
    # routed to 8 experts drawn by the decode routing generator
    c = wl.C3
    pr = next(p for p in c.projs if p.name == proj)
    qw = encode_stack(c, pr)
    ids_np = wl.decode_ids(c.cid, 0, c.E, 8)
    x = torch.randn(pr.K, generator=wl.torch_generator(DEV, c.cid, wl.T_X), device=DEV).to(torch.bfloat16)
    y = tq.gather_qmv(qw, torch.from_numpy(ids_np).to(DEV), x)
    torch.cuda.synchronize()
    yg, xf = as_f64(y), as_f64(x)
    g = wl.rng(c.cid, 90)
    for k, e in enumerate(ids_np):
        rows = np.sort(g.choice(pr.N, 48, replace=False))
        sampled_check(qw, int(e), rows, xf, yg[k, rows], f"C3 {proj} slot {k} expert {e}")


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_ternary_prefill_multi_gather_full_size(proj):
    # 128 experts, hidden 2048, intermediate 768, trits g16; 64 tokens routed top-8
    c = wl.C4
    pr = next(p for p in c.projs if p.name == proj)
    qw = encode_stack(c, pr)
    ids_np = wl.topk_routing(c.cid, 64, c.E, 8)
    P = len(ids_np)
    X = torch.randn((P, pr.K), generator=wl.torch_generator(DEV, c.cid, wl.T_X), device=DEV).to(torch.bfloat16)
    ws = torch.empty((tq.workspace_bytes(tq.OP_MULTI_GATHER_QMV, qw, P) + 7) // 8, dtype=torch.int64, device=DEV)
    y = tq.multi_gather_qmv(qw, torch.from_numpy(ids_np).to(DEV), X, ws=ws)
    torch.cuda.synchronize()
    yg, Xf = as_f64(y), as_f64(X)
    g = wl.rng(c.cid, 91)
    for p_ in np.sort(g.choice(P, 24, replace=False)):
        rows = np.sort(g.choice(pr.N, 32, replace=False))
        e = int(ids_np[p_])
        sampled_check(qw, e, rows, Xf[p_], yg[p_, rows], f"C4 {proj} pair {p_} expert {e}")


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_batched_gather_qmm_full_size(proj):
    # 4096 tokens x top-8 of 128 experts (Zipf-skewed), hidden 4096, intermediate 1536,
    # 4-bit g128; rows sorted by expert; gate reads the token rows, down one input per row
    c = wl.C5
    pr = next(p for p in c.projs if p.name == proj)
    qw = encode_stack(c, pr)
    T, k = 4096, 8
    row_token, row_expert, offsets = wl.zipf_sorted_routing(c.cid, T, c.E, k)
    M = len(row_token)
    gen = wl.torch_generator(DEV, c.cid, wl.T_X)
    if proj == "gate":
        X = torch.randn((T, pr.K), generator=gen, device=DEV).to(torch.bfloat16)
        rt = row_token
    else:
        X = torch.randn((M, pr.K), generator=gen, device=DEV).to(torch.bfloat16)
        rt = np.arange(M, dtype=np.int32)
    ws = torch.empty((tq.workspace_bytes(tq.OP_GATHER_QMM, qw, M, X.shape[0]) + 7) // 8,
                     dtype=torch.int64, device=DEV)
    y = tq.gather_qmm(qw, X, torch.from_numpy(rt).to(DEV), torch.from_numpy(offsets).to(DEV), ws=ws)
    torch.cuda.synchronize()
    g = wl.rng(c.cid, 92)
    ms = np.sort(g.choice(M, 40, replace=False))
    ys = as_f64(y[torch.from_numpy(ms).to(DEV)])
    Xs = as_f64(X[torch.from_numpy(rt[ms]).to(DEV)])
    for i, m in enumerate(ms):
        e = int(row_expert[m])
        assert offsets[e] <= m < offsets[e + 1]
        cols = np.sort(g.choice(pr.N, 48, replace=False))
        sampled_check(qw, e, cols, Xs[i], ys[i, cols], f"C5 {proj} row {m} expert {e}")


def test_dequant_full_size_gate_stack():
    # the whole batched-MoE gate stack (128 experts x 1536 x 4096, 4-bit g128) decoded to
    # bf16 in one call, as bench.py times it; sampled rows of sampled experts checked
    # against the oracle's fp64 dequantization of the GPU's own codes
    from oracle import encode as oenc
    c = wl.C5
    pr = c.projs[0]
    qw = encode_stack(c, pr)
    out = tq.dequant(qw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    g = wl.rng(c.cid, 93)
    for e in np.sort(g.choice(c.E, 6, replace=False)):
        rows = np.sort(g.choice(pr.N, 16, replace=False))
        codes = torch_to_np(qw.codes[int(e), rows]).reshape(len(rows), -1)
        scales = torch_to_np(qw.scales[int(e), rows]).reshape(len(rows), -1)
        want = oenc.dequant(codes, scales, pr.levels, pr.group, pr.K)
        got = as_f64(out[int(e), torch.from_numpy(rows).to(DEV)])
        tol = np.abs(want) * 2.0 ** -7
        assert np.all(np.abs(got - want) <= tol), f"expert {e}"


def test_full_size_pairs_equal_single_calls():
    # the gate/up pair calls of the three MoE workloads at full size, in the configuration
    # bench.py times: each half equals the one-weight call bit for bit, and sampled rows of
    # the second weight's half match the oracle
    g = wl.rng(93, 0)
    # MoE decode: gather_qmv_pair over 8 routed experts of 384
    c = wl.C3
    gate = encode_stack(c, c.projs[0])
    up = encode_stack(c, c.projs[1])
    ids = torch.from_numpy(wl.decode_ids(c.cid, 1, c.E, 8)).to(DEV)
    x = torch.randn(c.projs[0].K, generator=wl.torch_generator(DEV, c.cid, wl.T_X),
                    device=DEV).to(torch.bfloat16)
    y = tq.gather_qmv_pair(gate, up, ids, x)
    y1, y2 = tq.gather_qmv(gate, ids, x), tq.gather_qmv(up, ids, x)
    torch.cuda.synchronize()
    assert torch.equal(y[:8], y1) and torch.equal(y[8:], y2)
    yg, xf = as_f64(y), as_f64(x)
    for k in (0, 5):
        rows = np.sort(g.choice(up.N, 32, replace=False))
        sampled_check(up, int(ids[k]), rows, xf, yg[8 + k, rows], f"C3 up slot {k}")
    del gate, up, y, y1, y2
    # ternary prefill: multi_gather_qmv_pair over 512 pairs (both weights' items in one launch)
    c = wl.C4
    gate = encode_stack(c, c.projs[0])
    up = encode_stack(c, c.projs[1])
    ids_np = wl.topk_routing(c.cid, 64, c.E, 8)
    P = len(ids_np)
    ids = torch.from_numpy(ids_np).to(DEV)
    X = torch.randn((P, gate.K), generator=wl.torch_generator(DEV, c.cid, wl.T_X),
                    device=DEV).to(torch.bfloat16)
    y = tq.multi_gather_qmv_pair(gate, up, ids, X)
    y1, y2 = tq.multi_gather_qmv(gate, ids, X), tq.multi_gather_qmv(up, ids, X)
    torch.cuda.synchronize()
    assert torch.equal(y[:P], y1) and torch.equal(y[P:], y2)
    yg, Xf = as_f64(y), as_f64(X)
    for p_ in np.sort(g.choice(P, 8, replace=False)):
        rows = np.sort(g.choice(up.N, 24, replace=False))
        sampled_check(up, int(ids_np[p_]), rows, Xf[p_], yg[P + p_, rows], f"C4 up pair {p_}")
    del gate, up, y, y1, y2
    # batched MoE: gather_qmm_pair over 32,768 sorted rows
    c = wl.C5
    gate = encode_stack(c, c.projs[0])
    up = encode_stack(c, c.projs[1])
    T = 4096
    row_token, row_expert, offsets = wl.zipf_sorted_routing(c.cid, T, c.E, 8)
    M = len(row_token)
    X = torch.randn((T, gate.K), generator=wl.torch_generator(DEV, c.cid, wl.T_X),
                    device=DEV).to(torch.bfloat16)
    rt, off = torch.from_numpy(row_token).to(DEV), torch.from_numpy(offsets).to(DEV)
    y = tq.gather_qmm_pair(gate, up, X, rt, off)
    y1, y2 = tq.gather_qmm(gate, X, rt, off), tq.gather_qmm(up, X, rt, off)
    torch.cuda.synchronize()
    assert torch.equal(y[:M], y1) and torch.equal(y[M:], y2)
    for m in np.sort(g.choice(M, 6, replace=False)):
        cols = np.sort(g.choice(up.N, 32, replace=False))
        ym = as_f64(y[M + int(m)])
        sampled_check(up, int(row_expert[m]), cols, as_f64(X[int(row_token[m])]), ym[cols],
                      f"C5 up row {m}")
