"""Benchmark of the hot path on one MI355X: one JSON line on stdout.

Default workload (the dense decode layer): a bf16 4096 x 4096 weight with Student-t rows,
encoded to 3-bit Lloyd-Max codes with group-128 fp16 scales; one step = encode the weight
once + 1000 qmv calls on a batch-1 bf16 activation (N(0,1), 8 outlier channels x20). The
1000 calls cycle over 80 separately allocated copies of the packed weight (525 MB, twice
the 256 MB last-level cache), so every call streams its codes from HBM. Encode and the
1000 calls are each captured once in a HIP graph and replayed, so host launch overhead is
not in the timed region.

  metric  fused qmv HBM GB/s: algorithmic bytes (packed codes + fp16 scales + bf16
          activation = 6,561,792 B per call) of the step's 1000 calls / the step's time
  roofline.achieved  the same bytes per call / the average qmv launch duration, from HIP
          events around the qmv graph (includes the gaps between back-to-back kernels)
  roofline.traffic  HBM bytes per qmv launch from the FETCH_SIZE / WRITE_SIZE counter
          passes recorded in profiles/ (scaled by a copy kernel of known size); null
          when the kernel sources no longer match the ones those counters were taken on
  encode_mweights_per_s  16,777,216 weights / the encode time of a step
  encode  Mweights/s, GB/s and fraction of HBM peak of that encode (bytes = bf16 source +
          packed codes + fp16 scales, 2.39 B per weight) and of the MoE decode layer's
          gate stack (7168-wide rows: the 28-point Hadamard factor) and down stack, timed
          with HIP events around each encode call as the stacks are built
  gather_qmv  the MoE decode step (384 experts; gate, up, down of 8 routed experts): GB/s
          of the routed experts' codes + scales + inputs per step, fraction of HBM peak
  cpu_baseline  the fp64 oracle (numpy, one BLAS thread) on a bounded sample of the same
          layer, in the same unit; host_cpu_count and host_affinity give the host's logical
          CPUs and the ones this process may use (one is used)

Other workloads (--config 3, 4, 5, 6, 7, 8) time gather_qmv, multi_gather_qmv, gather_qmm,
dequant, the streamed encode from pinned host memory, the MoE decode with its experts
streamed from pinned host memory, the KV-cache fetch (--config 9) and a layer with a dense
rotation (--config 10), for reference; the default line is the dense decode layer.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_16BIT_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5, 6, 7, 8, 9, 10],
                    help="2 dense qmv (default), 3 gather_qmv, 4 multi_gather_qmv, "
                         "5 gather_qmm, 6 dequant of an expert stack, 7 encode of an "
                         "expert stack streamed from pinned host memory, 8 MoE decode with "
                         "its experts streamed from pinned host memory, 9 KV-cache fetch, "
                         "10 a layer with a dense (QR) rotation, K = 4864")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-moe", action="store_true",
                    help="default line without the MoE decode (gather_qmv) sub-measurement")
    ap.add_argument("--calls", type=int, default=1000, help="qmv calls per step")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 5 times (a plain copy kernel of "
                         "known size, to scale the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def cpu_baseline_qmv(W_bits, x_bits, levels, group, seed, budget_s=12.0, rows=512):
    """Oracle encode + qmv on the first `rows` rows of the layer; qmv timed, GB/s."""
    from threadpoolctl import threadpool_limits
    import numpy as np
    import workloads as wl
    from oracle import encode as oenc
    from oracle import ops as oops

    with threadpool_limits(limits=1):
        W = wl.bf16_bits_to_f64(W_bits[:rows])
        x = wl.bf16_bits_to_f64(x_bits)
        K = W.shape[1]
        t0 = time.perf_counter()
        ref = oenc.encode(W, levels, group, seed)
        t_enc = time.perf_counter() - t0
        n, t_q = 0, 0.0
        while t_q < budget_s and n < 50:
            t0 = time.perf_counter()
            oops.qmv(ref.codes, ref.scales, levels, group, K, seed, x)
            t_q += time.perf_counter() - t0
            n += 1
    nbytes = ref.codes.nbytes + ref.scales.nbytes + x_bits.nbytes
    return {
        "value": round(nbytes * n / t_q / 1e9, 6),
        "unit": "GB/s",
        "cores": 1,
        "host_cpu_count": os.cpu_count(),
        "host_affinity": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"oracle (numpy fp64, 1 BLAS thread) qmv of the first {rows} of 4096 rows "
                  f"of the layer, {n} calls in {t_q:.1f} s; oracle encode of those rows "
                  f"{rows * K / t_enc / 1e6:.3f} Mweights/s",
        "encode_mweights_per_s": round(rows * K / t_enc / 1e6, 6),
    }


QMV_SOURCES = ["qmv.hip", "qmv_16.hip", "qmv_8.hip", "qmv_4.hip", "qmv_3.hip", "qmv_kernel.hpp",
               "qmv_decode.hpp", "rot_mfma.hpp", "prologue.hpp", "decode_common.hpp",
               "fwht_block.hpp", "device_common.hpp", "internal.hpp"]


def recorded_traffic(profile, sources):
    """HBM bytes per launch measured by the FETCH_SIZE / WRITE_SIZE passes recorded in
    profiles/<profile>, or None when the kernel sources have changed since (sha256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = line.split(":", 1)
            rec[k] = v.strip()
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "rotation_lloyd_max_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if rec.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in rec:
        return None
    return int(rec["traffic_bytes_per_launch"])


def copy_calibration(mib):
    """Five device-to-device copies of `mib` MiB by an elementwise kernel (y = 1 * x, fp32)."""
    import torch
    n = mib << 20
    src = torch.rand(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}


def bench_dense(args):
    import numpy as np
    import torch

    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    c = wl.C2
    p = c.projs[0]
    N, K, L, G = p.N, p.K, p.levels, p.group
    W_bits = wl.f32_to_bf16_bits(wl.student_rows(wl.rng(c.cid, wl.T_W), N, K))
    x_bits = wl.f32_to_bf16_bits(wl.gaussian(wl.rng(c.cid, wl.T_X), 1, K, outliers=8)[0])
    W = torch.from_numpy(W_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    x = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).to(dev)

    ncopy = 80
    base = tq.encode(W, L, G, p.seed)
    copies = [base] + [tq.QWeight(base.codes.clone(), base.scales.clone(), base.signs, L, G, K,
                                  N, 1, p.seed) for _ in range(ncopy - 1)]
    y = torch.empty(N, dtype=torch.float32, device=dev)
    calls = args.calls

    def run_encode():
        tq.encode(W, L, G, p.seed, out=copies[0])

    def run_qmv():
        for i in range(calls):
            tq.qmv(copies[i % ncopy], x, out=y)

    # eager once (warms the library), then capture both phases
    run_encode()
    run_qmv()
    torch.cuda.synchronize()
    g_enc, g_qmv = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_enc):
        run_encode()
    with torch.cuda.graph(g_qmv):
        run_qmv()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        g_enc.replay()
        g_qmv.replay()
    torch.cuda.synchronize()

    steps = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        g_enc.replay()
        ev[s][1].record()
        g_qmv.replay()
        ev[s][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = sum(e[0].elapsed_time(e[1]) for e in ev)
    qmv_ms = sum(e[1].elapsed_time(e[2]) for e in ev)
    total_ms = ev[0][0].elapsed_time(ev[-1][2])
    ms_per_step = total_ms / steps

    bytes_call = (N * tq.words_per_row(K, L) * 4) + (N * (K // G) * 2) + K * 2
    value = bytes_call * calls / (ms_per_step / 1e3) / 1e9
    avg_qmv_s = qmv_ms / 1e3 / (steps * calls)
    achieved = bytes_call / avg_qmv_s / 1e9
    out = {
        "metric": "fused qmv HBM GB/s (dense decode layer, encode + 1000 cold qmv per step)",
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16*f16->f32 (decode), f64 (encode)",
        "data": "synthetic",
        "config": {
            "workload": "dense decode qmv: bf16 W 4096x4096 (Student-t df=4 x lognormal rows), "
                        "3-bit Lloyd-Max, group 128, fp16 scales; bf16 x N(0,1) + 8 outliers x20; "
                        "step = encode + 1000 qmv over 80 cold copies",
            "N": N, "K": K, "bits": 3, "group": G, "qmv_per_step": calls, "cold_copies": ncopy,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "bytes_per_qmv": bytes_call,
        "qmv_avg_us": round(avg_qmv_s * 1e6, 4),
        "encode_mweights_per_s": round(N * K / (enc_ms / 1e3 / steps) / 1e6, 3),
        "wall_s": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic("k_qmv_dense_4096x4096_3bit_g128.md", QMV_SOURCES),
        },
    }
    enc_rates = {"dense 4096x4096 bf16 -> 3-bit g128 (once per step)":
                 encode_rate(N * K * steps, enc_ms, 2, L, G)}
    del copies, base
    torch.cuda.empty_cache()
    if not args.no_moe:
        moe = moe_decode_measure(steps=max(20, args.steps * 2), warmup=args.warmup)
        for k, v in moe.pop("encode").items():
            enc_rates[k] = v
        out["gather_qmv"] = moe
    out["encode"] = enc_rates
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_qmv(W_bits, x_bits, L, G, p.seed)
    return out


def moe_decode_measure(steps, warmup):
    """The MoE decode layer (384 experts, hidden 7168, intermediate 2048; gate and up 2-bit
    g64, down 4-bit g64): every step routes one token to 8 experts drawn uniformly and runs
    gather_qmv_pair for gate and up (one launch: shared 7168-wide input, same ids, one
    rotation) and gather_qmv for down (2048-wide input). Steps are
    captured 20 to a graph with 20 different routings and timed with HIP events around the
    replays. Bytes per step = the 8 routed experts' codes and scales of the three
    projections + the bf16 inputs (128,450,560 + 32,768 B). Also returns the encode rates of
    the stacks as they are built (HIP events around each encode call)."""
    import numpy as np
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    c = wl.C3
    timing = {}
    layer = {}
    for pr in c.projs:
        t = [] if pr.name != "up" else None
        layer[pr.name] = encode_stack(c.E, pr.N, pr.K, pr.levels, pr.group, pr.seed, c.cid,
                                      wl.PROJ_TENSOR[pr.name], dev, timing=t)
        if t:
            timing[pr.name] = (pr, t[0])
    wbytes = {pr.name: layer[pr.name].codes.numel() * 4 // c.E +
              layer[pr.name].scales.numel() * 2 // c.E for pr in c.projs}
    per_graph = 20
    K1, K2 = c.projs[0].K, c.projs[2].K
    ids = torch.from_numpy(np.stack([wl.decode_ids(c.cid, s, c.E, 8)
                                     for s in range(per_graph)])).to(dev)
    x1 = torch.randn(K1, generator=wl.torch_generator(dev, c.cid, wl.T_X), device=dev).to(torch.bfloat16)
    x2 = torch.randn(K2, generator=wl.torch_generator(dev, c.cid, wl.T_XD), device=dev).to(torch.bfloat16)
    y_gu = torch.empty((16, c.projs[0].N), dtype=torch.float32, device=dev)  # gate; up
    y_down = torch.empty((8, c.projs[2].N), dtype=torch.float32, device=dev)

    def step(s):
        tq.gather_qmv_pair(layer["gate"], layer["up"], ids[s], x1, out=y_gu)
        tq.gather_qmv(layer["down"], ids[s], x2, out=y_down)

    for s in range(per_graph):
        step(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(per_graph):
            step(s)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // per_graph)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    nsteps = reps * per_graph
    ms_per_step = e0.elapsed_time(e1) / nsteps
    bytes_step = 8 * sum(wbytes.values()) + 2 * K1 * 2 + K2 * 2
    gbs = bytes_step / (ms_per_step / 1e3) / 1e9
    enc = {}
    for name, (pr, (w, ms)) in timing.items():
        key = (f"MoE {name} stack {c.E}x{pr.N}x{pr.K} bf16 -> "
               f"{ {4: '2-bit', 16: '4-bit'}[pr.levels]} g{pr.group}")
        enc[key] = encode_rate(w, ms, 2, pr.levels, pr.group)
    del layer
    torch.cuda.empty_cache()
    return {"metric": "gather_qmv HBM GB/s (MoE decode: gate+up+down of 8 routed experts)",
            "value": round(gbs, 3), "unit": "GB/s", "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "ms_per_step": round(ms_per_step, 6), "steps": nsteps, "bytes_per_step": bytes_step,
            "encode": enc}


def encode_stack(E, N, K, levels, group, seed, cfg, tensor, dev, chunk=16, timing=None):
    """Encode an expert stack whose bf16 weights are drawn on the GPU, chunk by chunk. With
    `timing` (a list), the encode calls alone are timed with HIP events on the current
    stream and (weights, milliseconds) is appended."""
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl
    wpr = tq.words_per_row(K, levels)
    codes = torch.empty((E, N, wpr), dtype=torch.int32, device=dev)
    scales = torch.empty((E, N, K // group), dtype=torch.float16, device=dev)
    sg = tq.signs(seed, K, dev)
    ms = 0.0
    if timing is not None:
        # one untimed call of the same shape first: the first launch of a kernel in a
        # process also loads its code
        g = wl.torch_generator(dev, cfg, tensor, 0)
        Wc = wl.torch_student_rows(g, min(chunk, E) * N, K, dev, torch.bfloat16).view(-1, N, K)
        part = tq.QWeight(codes[:Wc.shape[0]], scales[:Wc.shape[0]], sg, levels, group, K, N, Wc.shape[0], seed)
        tq.encode(Wc, levels, group, seed, out=part)
        del Wc
    for e0 in range(0, E, chunk):
        e1 = min(E, e0 + chunk)
        g = wl.torch_generator(dev, cfg, tensor, e0)
        Wc = wl.torch_student_rows(g, (e1 - e0) * N, K, dev, torch.bfloat16).view(e1 - e0, N, K)
        part = tq.QWeight(codes[e0:e1], scales[e0:e1], sg, levels, group, K, N, e1 - e0, seed)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        tq.encode(Wc, levels, group, seed, out=part)
        b.record()
        if timing is not None:
            b.synchronize()
            ms += a.elapsed_time(b)
        del Wc
    torch.cuda.synchronize()
    if timing is not None:
        timing.append((E * N * K, ms))
    return tq.QWeight(codes, scales, sg, levels, group, K, N, E, seed)


def encode_rate(weights, ms, src_bytes, levels, group):
    """Encode throughput and its HBM fraction: bytes = source + packed codes + fp16 scales."""
    bits = {3: 1.6, 4: 2, 8: 3, 16: 4}[levels]
    per_w = src_bytes + bits / 8 + 2.0 / group
    gbs = weights * per_w / (ms / 1e3) / 1e9
    return {"mweights_per_s": round(weights / (ms / 1e3) / 1e6, 3), "bytes_per_weight": per_w,
            "gb_per_s": round(gbs, 3), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def bench_moe(args):
    """gather_qmv (3), multi_gather_qmv (4) or gather_qmm (5) on the full expert stacks."""
    import numpy as np
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    c = wl.CONFIGS[args.config]
    if args.config == 3:
        m = moe_decode_measure(args.steps, args.warmup)
        return {
            "metric": m["metric"], "value": m["value"], "unit": "GB/s", "n_gpus": 1,
            "steps": m["steps"], "warmup": args.warmup, "ms_per_step": m["ms_per_step"],
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "f16*f16->f32", "data": "synthetic",
            "config": {"workload": c.name, "bytes_per_step": m["bytes_per_step"]},
            "roofline": {"bound": "hbm", "achieved": m["value"], "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": m["frac_of_hbm_peak"], "traffic": None},
            "encode": m["encode"],
        }
    ncopy = 3 if args.config == 4 else 1
    layers = []
    for _ in range(ncopy):
        layers.append({pr.name: encode_stack(c.E, pr.N, pr.K, pr.levels, pr.group, pr.seed,
                                             c.cid, wl.PROJ_TENSOR[pr.name], dev)
                       for pr in c.projs})
    wbytes = {pr.name: layers[0][pr.name].codes.numel() * 4 // c.E +
              layers[0][pr.name].scales.numel() * 2 // c.E for pr in c.projs}
    steps_per_graph = 20
    if args.config == 4:
        P = 64 * 8
        ids_np = wl.topk_routing(c.cid, 64, c.E, 8)
        ids = torch.from_numpy(ids_np).to(dev)
        Kg, Kd = c.projs[0].K, c.projs[2].K
        g = wl.torch_generator(dev, c.cid, wl.T_X)
        # a pair's input is its token's row, read by gate and up; down reads its own rows
        xg = torch.randn((P, Kg), generator=g, device=dev).to(torch.bfloat16)
        xd = torch.randn((P, Kd), generator=g, device=dev).to(torch.bfloat16)
        y_gu = torch.empty((2 * P, c.projs[0].N), dtype=torch.float32, device=dev)  # gate; up
        y_d = torch.empty((P, c.projs[2].N), dtype=torch.float32, device=dev)
        wss = {pr.name: torch.empty((tq.workspace_bytes(tq.OP_MULTI_GATHER_QMV, layers[0][pr.name], P) + 7) // 8,
                                    dtype=torch.int64, device=dev) for pr in c.projs}

        def step(s):
            L = layers[s % ncopy]
            tq.multi_gather_qmv_pair(L["gate"], L["up"], ids, xg, out=y_gu, ws=wss["gate"])
            tq.multi_gather_qmv(L["down"], ids, xd, out=y_d, ws=wss["down"])
        touched = len(np.unique(ids_np))
        bytes_step = touched * sum(wbytes.values()) + (xg.numel() + xd.numel()) * 2
        unit, metric = "GB/s", "multi_gather_qmv HBM GB/s (ternary MoE prefill: gate+up+down)"
    else:
        T, k = 4096, 8
        row_token, _, offsets = wl.zipf_sorted_routing(c.cid, T, c.E, k)
        M = len(row_token)
        rt = torch.from_numpy(row_token).to(dev)
        off = torch.from_numpy(offsets).to(dev)
        ident = torch.arange(M, dtype=torch.int32, device=dev)
        Kg, Kd = c.projs[0].K, c.projs[2].K
        g = wl.torch_generator(dev, c.cid, wl.T_X)
        x = torch.randn((T, Kg), generator=g, device=dev).to(torch.bfloat16)
        xd = torch.randn((M, Kd), generator=g, device=dev).to(torch.bfloat16)
        ys = {"down": torch.empty((M, c.projs[2].N), dtype=torch.bfloat16, device=dev)}
        wsg = torch.empty((tq.workspace_bytes(tq.OP_GATHER_QMM, layers[0]["gate"], M, T) + 7) // 8,
                          dtype=torch.int64, device=dev)
        wsd = torch.empty((tq.workspace_bytes(tq.OP_GATHER_QMM, layers[0]["down"], M, M) + 7) // 8,
                          dtype=torch.int64, device=dev)
        steps_per_graph = 1

        y_gu = torch.empty((2 * M, c.projs[0].N), dtype=torch.bfloat16, device=dev)  # gate; up

        def step(s):
            L = layers[0]
            tq.gather_qmm_pair(L["gate"], L["up"], x, rt, off, out=y_gu, ws=wsg)
            tq.gather_qmm(L["down"], xd, ident, off, out=ys["down"], ws=wsd)
        flops_step = 2.0 * M * (2 * Kg * c.projs[0].N + Kd * c.projs[2].N)
        bytes_step = c.E * sum(wbytes.values())
        unit, metric = "TFLOP/s", "gather_qmm TFLOP/s on 16-bit matrix cores (batched MoE: gate+up+down)"

    for s in range(steps_per_graph):
        step(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(steps_per_graph):
            step(s)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // steps_per_graph) if steps_per_graph > 1 else args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nsteps = reps * steps_per_graph
    ms_per_step = e0.elapsed_time(e1) / nsteps
    if args.config == 5:
        value = flops_step / (ms_per_step / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(value, 3), "peak": MFMA_16BIT_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(value / MFMA_16BIT_PEAK_TFLOPS, 4), "traffic": None}
    else:
        value = bytes_step / (ms_per_step / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(value, 3), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None}
    return {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": nsteps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 MFMA, f32 acc" if args.config == 5 else "f16*f16->f32",
        "data": "synthetic", "config": {"workload": c.name, "bytes_per_step": bytes_step},
        "wall_s": round(wall, 4), "roofline": roof,
    }


def bench_dequant(args):
    """dequant of the batched-MoE gate stack (128 experts x 1536 x 4096, 4-bit g128) to bf16:
    codes and scales read once, the decoded weights written once, per step."""
    import numpy as np
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    c = wl.C5
    pr = c.projs[0]
    qw = encode_stack(c.E, pr.N, pr.K, pr.levels, pr.group, pr.seed, c.cid,
                      wl.PROJ_TENSOR[pr.name], dev)
    out = torch.empty((c.E, pr.N, pr.K), dtype=torch.bfloat16, device=dev)
    tq.dequant(qw, out=out)
    torch.cuda.synchronize()
    # several calls per graph, so that the launch gap of a replay is paid once per group
    steps_per_graph = 5
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps_per_graph):
            tq.dequant(qw, out=out)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // steps_per_graph)
    nsteps = reps * steps_per_graph
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / nsteps
    read = qw.codes.numel() * 4 + qw.scales.numel() * 2
    written = out.numel() * 2
    value = (read + written) / (ms / 1e3) / 1e9
    res = {
        "metric": "dequant HBM GB/s (expert stack to bf16: codes and scales read, weights "
                  "written)",
        "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": nsteps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 product -> bf16",
        "data": "synthetic",
        "config": {"workload": "dequant of the batched-MoE gate stack: 128 experts x 1536 x "
                               "4096, 4-bit Lloyd-Max g128 -> bf16", "bytes_per_step": read + written},
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(value, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_limits
        from oracle import encode as oenc
        codes = qw.codes[0].cpu().numpy().view(np.uint32)
        scales = qw.scales[0].view(torch.int16).cpu().numpy().view(np.uint16)
        with threadpool_limits(1):
            t = time.perf_counter()
            n = 0
            while n == 0 or time.perf_counter() - t < 10.0:
                oenc.dequant(codes, scales, pr.levels, pr.group, pr.K)
                n += 1
            dt = (time.perf_counter() - t) / n
        b1 = codes.size * 4 + scales.size * 2 + pr.N * pr.K * 2
        res["cpu_baseline"] = {"value": round(b1 / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"oracle (numpy fp64, 1 BLAS thread) dequant of expert 0 "
                                         f"({pr.N} x {pr.K}), {n} calls in {dt * n:.1f} s"}
    return res


def bench_encode_stream(args):
    """encode_stream of 16 experts of the batched-MoE gate stack (16 x 1536 x 4096 bf16,
    201 MB) from pinned host memory through a 64 MB device staging buffer, copies on their
    own stream: host bytes per second, PCIe included (the input is not in HBM)."""
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    c = wl.C5
    pr = c.projs[0]
    E = 16
    g = wl.torch_generator(dev, c.cid, wl.PROJ_TENSOR[pr.name], 0)
    Wd = wl.torch_student_rows(g, E * pr.N, pr.K, dev, torch.bfloat16).view(E, pr.N, pr.K)
    W = torch.empty(Wd.shape, dtype=torch.bfloat16, pin_memory=True)
    W.copy_(Wd)
    ref = tq.encode(Wd, pr.levels, pr.group, pr.seed)
    del Wd
    torch.cuda.synchronize()
    out = tq.QWeight(torch.empty_like(ref.codes), torch.empty_like(ref.scales), ref.signs,
                     pr.levels, pr.group, pr.K, pr.N, E, pr.seed)
    cs = torch.cuda.Stream(device=dev)
    staging = 64 << 20

    def call():
        tq.encode_stream(W, pr.levels, pr.group, pr.seed, device=dev, staging_bytes=staging,
                         out=out, copy_stream=cs)

    call()
    torch.cuda.synchronize()
    same = torch.equal(out.codes, ref.codes) and torch.equal(out.scales.view(torch.int16),
                                                           ref.scales.view(torch.int16))
    if not same:
        raise RuntimeError("encode_stream differs from encode")
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(args.steps):
        call()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / args.steps
    host = W.numel() * 2
    value = host / (ms / 1e3) / 1e9
    return {
        "metric": "encode_stream GB/s of host weight bytes (pinned host -> HBM, PCIe included)",
        "value": round(value, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, f64 rotation",
        "data": "synthetic",
        "config": {"workload": "encode_stream of 16 experts of the batched-MoE gate stack "
                               "(16 x 1536 x 4096 bf16, 4-bit g128), 64 MB staging",
                   "bytes_per_step": host, "byte_identical_to_encode": same},
        "wall_s": round(wall, 4),
    }


def bench_expert_stream(args):
    """The MoE decode layer with its experts streamed from pinned host memory: gate, up and
    down stacks (384 experts each, 6.2 GB) stay on the host, 64 device slots per projection
    hold the experts in use (least recently used out), and each step fetches the 8 routed
    experts (uniform routing) before its three gather_qmv calls. Reported: step time, the
    host-to-device bytes of the step's copies (PCIe included), and the hit rate."""
    import numpy as np
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    c = wl.C3
    slots = 64
    caches, copy = {}, torch.cuda.Stream(device=dev)
    per_expert = {}
    for pr in c.projs:
        qw = encode_stack(c.E, pr.N, pr.K, pr.levels, pr.group, pr.seed, c.cid,
                          wl.PROJ_TENSOR[pr.name], dev)
        host = tq.QWeight(qw.codes.cpu().pin_memory(), qw.scales.cpu().pin_memory(), qw.signs,
                          pr.levels, pr.group, pr.K, pr.N, c.E, pr.seed)
        per_expert[pr.name] = qw.codes[0].numel() * 4 + qw.scales[0].numel() * 2
        del qw
        torch.cuda.empty_cache()
        caches[pr.name] = tq.ExpertCache(host, slots, copy_stream=copy)
    K1, K2 = c.projs[0].K, c.projs[2].K
    x1 = torch.randn(K1, generator=wl.torch_generator(dev, c.cid, wl.T_X), device=dev).to(torch.bfloat16)
    x2 = torch.randn(K2, generator=wl.torch_generator(dev, c.cid, wl.T_XD), device=dev).to(torch.bfloat16)
    ys = {pr.name: torch.empty((8, pr.N), dtype=torch.float32, device=dev) for pr in c.projs}
    total = args.warmup + args.steps
    routes = [wl.decode_ids(c.cid, s, c.E, 8) for s in range(total)]

    def step(s):
        moved = 0
        for name, x in (("gate", x1), ("up", x1), ("down", x2)):
            sid, n = caches[name].fetch(routes[s])
            tq.gather_qmv(caches[name].pool, sid, x, out=ys[name])
            moved += n * per_expert[name]
        return moved

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    moved = sum(step(args.warmup + s) for s in range(args.steps))
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = a.elapsed_time(b) / args.steps
    hits = sum(cch.stats()[0] for cch in caches.values())
    misses = sum(cch.stats()[1] for cch in caches.values())
    gbs = moved / args.steps / (ms / 1e3) / 1e9
    return {
        "metric": "streamed MoE decode: host-to-device GB/s of expert copies (PCIe included)",
        "value": round(gbs, 3), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16*f16->f32", "data": "synthetic",
        "config": {"workload": c.name + "; experts in pinned host memory, 64 device slots per "
                               "projection, uniform routing", "slots": slots,
                   "bytes_copied_per_step": moved // args.steps},
        "hit_rate": round(hits / max(1, hits + misses), 4), "wall_s": round(wall, 4),
    }


def bench_kv(args):
    """KV-cache compression: a cache of 32,768 tokens x 8 KV heads x head_dim 128 with 8-bit
    keys and 3-bit values (groups of 64), stored with tq_encode; one step fetches the whole
    cache (both halves dequantized and rotated back to bf16), as a decode step that reads
    every cached key and value would. Bytes per step = packed codes + fp16 scales read +
    bf16 rows written. The store rate of the whole cache is reported beside it."""
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    T, H, d, g = 32768, 8, 128, 64
    gen = wl.torch_generator(dev, 9, wl.T_X)
    ch = torch.randperm(d, generator=torch.Generator().manual_seed(9))[:4]
    Kx = torch.randn((T * H, d), generator=gen, device=dev)
    Kx[:, ch.to(dev)] *= 20.0  # fixed outlier channels of attention keys
    Kx = Kx.to(torch.bfloat16)
    Vx = torch.randn((T * H, d), generator=gen, device=dev).to(torch.bfloat16)
    kq = tq.encode(Kx, 256, g, 0)
    vq = tq.encode(Vx, 8, g, 1)
    ko = torch.empty((1, T * H, d), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    torch.cuda.synchronize()

    def store():
        tq.encode(Kx, 256, g, 0, out=kq)
        tq.encode(Vx, 8, g, 1, out=vq)

    def fetch():
        tq.kv_fetch(kq, out=ko)
        tq.kv_fetch(vq, out=vo)

    per_graph = 5
    gs, gf = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    store(); fetch()
    torch.cuda.synchronize()
    with torch.cuda.graph(gs):
        store()
    with torch.cuda.graph(gf):
        for _ in range(per_graph):
            fetch()
    for _ in range(args.warmup):
        gs.replay(); gf.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // per_graph)
    a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    t0 = time.perf_counter()
    a.record()
    for _ in range(reps):
        gf.replay()
    b.record()
    for _ in range(reps):
        gs.replay()
    c.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    nsteps = reps * per_graph
    ms = a.elapsed_time(b) / nsteps
    store_ms = b.elapsed_time(c) / reps
    read = (kq.codes.numel() + vq.codes.numel()) * 4 + (kq.scales.numel() + vq.scales.numel()) * 2
    written = (ko.numel() + vo.numel()) * 2
    gbs = (read + written) / (ms / 1e3) / 1e9
    src = (Kx.numel() + Vx.numel()) * 2
    store_gbs = (src + read) / (store_ms / 1e3) / 1e9
    return {
        "metric": "KV-cache fetch HBM GB/s (8-bit keys + 3-bit values dequantized and rotated back to bf16)",
        "value": round(gbs, 3), "unit": "GB/s", "n_gpus": 1, "steps": nsteps,
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 decode -> bf16", "data": "synthetic",
        "config": {"workload": "KV cache 32768 tokens x 8 heads x 128, keys 8-bit g64 (4 outlier "
                               "channels x20), values 3-bit g64; step = fetch of the whole cache",
                   "bytes_per_step": read + written},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "store": {"ms": round(store_ms, 6), "gb_per_s": round(store_gbs, 3),
                  "tokens_per_s": round(T / (store_ms / 1e3), 1)},
        "wall_s": round(wall, 4),
    }


def bench_dense_rotation(args):
    """A layer whose input dimension has no Hadamard matrix (K = 4864 = 19 x 256, the
    dimension VeloxQuant-MLX falls back to a QR rotation for): W 4096 x 4864 bf16, a Haar
    rotation R (4864 x 4864 fp32, 95 MB), 3-bit g128. Timed: the encode (R applied on the
    fp64 matrix cores, then snap and pack), R applied to one token (the whole matrix read
    per token) and to a batch of 4096 tokens, and one pre-rotated qmv."""
    import numpy as np
    import torch
    import rotation_lloyd_max_amd as tq
    import workloads as wl

    dev = torch.device("cuda:0")
    N, K, L, G = 4096, 4864, 8, 128
    R = torch.from_numpy(np.array(wl.haar_rotation(K, 1))).to(dev)
    gen = wl.torch_generator(dev, 10, wl.T_W)
    W = wl.torch_student_rows(gen, N, K, dev, torch.bfloat16)
    x1 = torch.randn((1, K), generator=gen, device=dev).to(torch.bfloat16)
    xb = torch.randn((4096, K), generator=gen, device=dev).to(torch.bfloat16)
    qw = tq.encode_dense(W, R, L, G)
    y1 = torch.empty((1, K), dtype=torch.float32, device=dev)
    yb = torch.empty((4096, K), dtype=torch.bfloat16, device=dev)
    out = torch.empty(N, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    enc_ms = timed(lambda: tq.encode_dense(W, R, L, G, out=qw), max(2, args.steps // 5))
    r1_ms = timed(lambda: tq.rotate_dense(x1, R, out=y1), args.steps)
    rb_ms = timed(lambda: tq.rotate_dense(xb, R, out=yb), max(2, args.steps // 5))
    q_ms = timed(lambda: tq.qmv(qw, y1[0], rotated=True, out=out), args.steps)
    fl_enc = 2.0 * N * K * K
    fl_b = 2.0 * 4096 * K * K
    return {
        "metric": "dense-rotation layer (K = 4864): encode and batch rotation on fp64 matrix cores, TFLOP/s",
        "value": round(fl_enc / (enc_ms / 1e3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": 1, "ms_per_step": round(enc_ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f64 MFMA (rotation), f16*f16->f32 (qmv)", "data": "synthetic",
        "config": {"workload": "W 4096 x 4864 bf16, Haar rotation 4864 x 4864 fp32, 3-bit g128"},
        "roofline": {"bound": "mfma", "achieved": round(fl_enc / (enc_ms / 1e3) / 1e12, 3),
                     "peak": 78.6, "unit": "TFLOP/s",
                     "frac": round(fl_enc / (enc_ms / 1e3) / 1e12 / 78.6, 4), "traffic": None},
        "encode_ms": round(enc_ms, 4),
        "rotate_one_token_us": round(r1_ms * 1e3, 3),
        "rotate_one_token_gb_per_s_of_R": round(K * K * 4 / (r1_ms / 1e3) / 1e9, 3),
        "rotate_4096_tokens_ms": round(rb_ms, 4),
        "rotate_4096_tokens_tflops": round(fl_b / (rb_ms / 1e3) / 1e12, 3),
        "qmv_pre_rotated_us": round(q_ms * 1e3, 3),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library has "
              "no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import rotation_lloyd_max_amd as tq
    if not os.path.exists(tq.LIB_PATH):
        from rotation_lloyd_max_amd import build
        build.build()
    if args.copy_calibration:
        out = copy_calibration(args.copy_calibration)
    elif args.config == 2:
        out = bench_dense(args)
    elif args.config == 6:
        out = bench_dequant(args)
    elif args.config == 7:
        out = bench_encode_stream(args)
    elif args.config == 8:
        out = bench_expert_stream(args)
    elif args.config == 9:
        out = bench_kv(args)
    elif args.config == 10:
        out = bench_dense_rotation(args)
    else:
        out = bench_moe(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
