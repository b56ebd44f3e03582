"""Expert streaming (tq_expert_cache_*): experts held in host memory, a few device slots,
least-recently-used replacement. Every output must be bit-identical to the same layer call
on the whole weight in device memory ("Expert streaming" of turboquant-mlx "How it works"),
and the slots chosen must follow the documented policy (a Python model of it below)."""

import numpy as np
import pytest
import torch

import rotation_lloyd_max_amd as tq
import workloads as wl
from test_gpu_encode import to_dev

pytestmark = pytest.mark.gpu


class LruModel:
    """The documented policy: hits keep their slot; each miss takes the least recently used
    slot that the call does not need (the lowest such slot on ties)."""

    def __init__(self, slots):
        self.slot_expert = [-1] * slots
        self.slot_tick = [0] * slots
        self.where = {}
        self.tick = 0

    def fetch(self, ids):
        self.tick += 1
        for e in ids:
            if e in self.where:
                self.slot_tick[self.where[e]] = self.tick
        out, copied = [], 0
        for e in ids:
            if e not in self.where:
                free = [s for s in range(len(self.slot_tick)) if self.slot_tick[s] != self.tick]
                s = min(free, key=lambda c: (self.slot_tick[c], c))
                if self.slot_expert[s] >= 0:
                    del self.where[self.slot_expert[s]]
                self.slot_expert[s] = e
                self.where[e] = s
                self.slot_tick[s] = self.tick
                copied += 1
            out.append(self.where[e])
        return out, copied


def host_copy(qw):
    """The same packed weight with codes and scales in pinned host memory."""
    return tq.QWeight(qw.codes.cpu().pin_memory(), qw.scales.cpu().pin_memory(), qw.signs,
                      qw.levels, qw.group, qw.K, qw.N, qw.E, qw.seed)


def stack(levels, group, K, E, N, seed):
    W = to_dev(wl.student_rows(wl.rng(985, levels, K), E * N, K), torch.bfloat16).view(E, N, K)
    return tq.encode(W, levels, group, seed)


def routings(g, E, steps, k):
    # a skewed popularity so that later steps find some experts resident
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    out = [g.choice(E, k, replace=False, p=p).astype(np.int32) for _ in range(steps)]
    out[3] = np.array([out[2][0], out[2][0], out[2][1]], dtype=np.int32)  # repeats in one call
    return out


@pytest.mark.parametrize("own_copy_stream", [True, False])
def test_streamed_gather_qmv_is_bit_identical(own_copy_stream):
    # MoE decode shapes (2-bit g64, K = 7168), 40 experts, 6 slots, 14 steps of 5 experts
    levels, group, K, E, N, slots = 4, 64, 7168, 40, 256, 6
    full = stack(levels, group, K, E, N, 0)
    cache = tq.ExpertCache(host_copy(full), slots,
                           copy_stream=torch.cuda.Stream() if own_copy_stream else None)
    model = LruModel(slots)
    g = wl.rng(986, 0)
    x = to_dev(wl.gaussian(g, 1, K)[0], torch.bfloat16)
    total_copied, total_ids = 0, 0
    for step, ids in enumerate(routings(g, E, 14, 5)):
        total_ids += len(ids)
        sid, copied = cache.fetch(ids)
        y = tq.gather_qmv(cache.pool, sid, x)
        y_full = tq.gather_qmv(full, torch.from_numpy(ids).cuda(), x)
        torch.cuda.synchronize()
        want_slots, want_copied = model.fetch(list(ids))
        assert sid.cpu().tolist() == want_slots, step
        assert copied == want_copied, step
        total_copied += copied
        assert torch.equal(y, y_full), f"step {step}"
    hits, misses = cache.stats()
    assert misses == total_copied and hits + misses == total_ids


def test_streamed_multi_gather_is_bit_identical():
    # ternary prefill shapes (g16, K = 2048): pairs over at most 5 distinct experts per call
    levels, group, K, E, N, slots = 3, 16, 2048, 20, 192, 5
    full = stack(levels, group, K, E, N, 0)
    cache = tq.ExpertCache(host_copy(full), slots, copy_stream=torch.cuda.Stream())
    g = wl.rng(987, 0)
    for step in range(8):
        experts = g.choice(E, 5, replace=False)
        ids = experts[g.integers(0, 5, 24)].astype(np.int32)
        X = to_dev(wl.gaussian(g, 24, K), torch.bfloat16)
        y = cache.multi_gather_qmv(ids, X)
        y_full = tq.multi_gather_qmv(full, torch.from_numpy(ids).cuda(), X)
        torch.cuda.synchronize()
        assert torch.equal(y, y_full), f"step {step}"


def test_fetch_errors_leave_the_cache_unchanged():
    levels, group, K, E, N, slots = 16, 64, 1024, 12, 64, 3
    full = stack(levels, group, K, E, N, 1)
    cache = tq.ExpertCache(host_copy(full), slots)
    model = LruModel(slots)
    for ids, ok in (([1, 2], True), ([0, 3, 4, 5], False), ([7, 12], False), ([2, 9, 1], True),
                    ([-1], False), ([5, 5, 5, 5, 6], True)):
        if not ok:
            with pytest.raises(tq.TqError):
                cache.fetch(ids)
            continue
        sid, copied = cache.fetch(ids)
        torch.cuda.synchronize()
        assert (sid.cpu().tolist(), copied) == model.fetch(ids)
