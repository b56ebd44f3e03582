"""The whole path captured once in a HIP graph (through torch.cuda.graph) and replayed with
new inputs: every replay must give bit for bit what the same calls give eagerly on those
inputs. The library records no memset and no allocation of its own; its workspaces come
from the caller (here torch's graph pool)."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from test_gpu_encode import to_dev

pytestmark = pytest.mark.gpu

E, N, K, LEVELS, GROUP, SEED = 4, 96, 1536, 16, 64, 5
P, T = 9, 24


def empty_weight(dev):
    wpr = tq.words_per_row(K, LEVELS)
    return tq.QWeight(torch.empty((E, N, wpr), dtype=torch.int32, device=dev),
                      torch.empty((E, N, K // GROUP), dtype=torch.float16, device=dev),
                      tq.signs(SEED, K, dev), LEVELS, GROUP, K, N, E, SEED)


def outputs(dev, M):
    return {"qw": empty_weight(dev),
            "qw2": empty_weight(dev),
            "qmv": torch.empty(N, dtype=torch.float32, device=dev),
            "gather": torch.empty((4, N), dtype=torch.bfloat16, device=dev),
            "gather_pair": torch.empty((8, N), dtype=torch.float32, device=dev),
            "multi": torch.empty((P, N), dtype=torch.float32, device=dev),
            "multi_pair": torch.empty((2 * P, N), dtype=torch.float32, device=dev),
            "qmm": torch.empty((M, N), dtype=torch.float16, device=dev),
            "dequant": torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)}


def test_graph_replays_match_eager():
    dev = torch.device("cuda")
    g = wl.rng(950, 0)
    Wb = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    Wb2 = torch.empty((E, N, K), dtype=torch.bfloat16, device=dev)
    x = torch.empty(K, dtype=torch.bfloat16, device=dev)
    X = torch.empty((P, K), dtype=torch.bfloat16, device=dev)
    Xq = torch.empty((T, K), dtype=torch.bfloat16, device=dev)
    ids = torch.tensor([2, 0, 3, 2], dtype=torch.int32, device=dev)
    pids = torch.from_numpy(g.integers(0, E, P).astype(np.int32)).to(dev)
    rt_np, _, off_np = wl.zipf_sorted_routing(950, T, E, 2)
    rt, off = torch.from_numpy(rt_np).to(dev), torch.from_numpy(off_np).to(dev)
    M = rt.numel()

    def fill(rep):
        r = wl.rng(951, rep)
        Wb.copy_(to_dev(wl.student_rows(r, E * N, K), torch.bfloat16).view(E, N, K))
        Wb2.copy_(to_dev(wl.student_rows(r, E * N, K), torch.bfloat16).view(E, N, K))
        x.copy_(to_dev(wl.gaussian(r, 1, K)[0], torch.bfloat16))
        X.copy_(to_dev(wl.gaussian(r, P, K), torch.bfloat16))
        Xq.copy_(to_dev(wl.gaussian(r, T, K, outliers=4), torch.bfloat16))

    def run(o):
        tq.encode(Wb, LEVELS, GROUP, SEED, out=o["qw"])
        q = o["qw"]
        one = tq.QWeight(q.codes[2:3], q.scales[2:3], q.signs, LEVELS, GROUP, K, N, 1, SEED)
        tq.qmv(one, x, out=o["qmv"])
        tq.gather_qmv(o["qw"], ids, x, out=o["gather"])
        tq.encode(Wb2, LEVELS, GROUP, SEED, out=o["qw2"])
        tq.gather_qmv_pair(o["qw"], o["qw2"], ids, x, out=o["gather_pair"])
        tq.multi_gather_qmv(o["qw"], pids, X, out=o["multi"])
        tq.multi_gather_qmv_pair(o["qw"], o["qw2"], pids, X, out=o["multi_pair"])
        tq.gather_qmm(o["qw"], Xq, rt, off, out=o["qmm"])
        tq.dequant(o["qw"], out=o["dequant"])

    og, oe = outputs(dev, M), outputs(dev, M)
    fill(0)
    run(og)  # eager once before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(og)
    torch.cuda.synchronize()
    for rep in range(1, 4):
        fill(rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        run(oe)
        torch.cuda.synchronize()
        assert torch.equal(og["qw"].codes, oe["qw"].codes), rep
        assert torch.equal(og["qw"].scales, oe["qw"].scales), rep
        for k in ("qmv", "gather", "gather_pair", "multi", "multi_pair", "qmm", "dequant"):
            assert torch.isfinite(oe[k]).all(), (rep, k)
            assert torch.equal(og[k], oe[k]), (rep, k)
    # the replays saw new inputs: the last results differ from the first ones
    fill(0)
    run(oe)
    torch.cuda.synchronize()
    assert not torch.equal(og["qmv"], oe["qmv"])
