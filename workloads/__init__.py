"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method (no rotation, no codebook, no packing): it
only draws weights, activations and routings, and rounds them to the storage dtype that
both the HIP library and the oracle then read byte for byte.

Weights: Student-t (4 degrees of freedom) entries times a per-row lognormal(0, 0.5) scale,
which gives the heavy tails and row-to-row spread of trained weight matrices; the method's
rotation is what makes such rows Gaussian ("How it works", "Quantizing a weight, with no
data"). Activations: N(0, 1), optionally with a few outlier channels. The MoE routings
mimic their decode / prefill / batched shapes ("Running a quantized layer", kernel table).

Seeds: numpy Generator(SeedSequence([config, tensor, expert])). Large expert stacks are
drawn on the GPU with a torch generator seeded the same way; the CPU-side checks read those
exact bytes back.
"""

from dataclasses import dataclass, field
from functools import lru_cache

import numpy as np

# tensor ids inside a config
T_W, T_X, T_ROUTE, T_GATE, T_UP, T_DOWN, T_XD = 0, 1, 2, 3, 4, 5, 6


def rng(config, tensor, expert=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([config, tensor, expert])))


def f32_to_bf16_bits(a):
    """Round float32 to bfloat16 (nearest even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def student_rows(g, rows, K):
    """fp32 [rows, K]: t(df=4) entries times a lognormal(0, 0.5) scale per row."""
    W = g.standard_t(4, size=(rows, K)) * np.exp(g.normal(0.0, 0.5, size=(rows, 1)))
    return W.astype(np.float32)


def gaussian(g, rows, K, outliers=0, factor=20.0):
    """fp32 [rows, K] N(0,1); `outliers` distinct channels (same for every row) scaled."""
    x = g.standard_normal((rows, K)).astype(np.float32)
    if outliers:
        ch = g.choice(K, outliers, replace=False)
        x[:, ch] *= factor
    return x


@lru_cache(maxsize=8)
def haar_rotation(K, seed):
    """A random K x K rotation from a seeded Gaussian matrix G: the orthogonal factor Q of
    G = Q R with the signs of R's diagonal moved into Q (Q diag(sign(diag R))), which makes Q
    Haar-distributed; rounded to float32, the form both sides read. This is the rotation's
    random draw (the QR-derived rotation of VeloxQuant-MLX), generated here like every
    other seeded input."""
    G = np.random.Generator(np.random.PCG64(np.random.SeedSequence([77, K, seed]))).standard_normal((K, K))
    Q, Rr = np.linalg.qr(G)
    Q = Q * np.sign(np.diag(Rr))[None, :]
    Q = Q.astype(np.float32)
    Q.flags.writeable = False  # cached: shared by every caller
    return Q


def kv_rows(g, tokens, heads, d, outliers=4, factor=20.0):
    """fp32 [tokens * heads, d]: N(0,1) head vectors (token-major, then head), with
    `outliers` channels of every head scaled by `factor` in every token: the fixed
    large-magnitude channels attention keys are known for, which give the raw vectors a
    heavy-tailed distribution that the rotation then spreads."""
    x = g.standard_normal((tokens, heads, d)).astype(np.float32)
    for h in range(heads):
        ch = g.choice(d, outliers, replace=False)
        x[:, h, ch] *= factor
    return x.reshape(tokens * heads, d)


def torch_student_rows(gen, rows, K, device, dtype):
    """Same distribution as student_rows, drawn on the GPU with a seeded torch generator:
    t(4) = Z / sqrt(chi2_4 / 4) with chi2_4 the sum of four squared normals."""
    import torch
    z = torch.randn((rows, K), generator=gen, device=device)
    c = torch.randn((4, rows, K), generator=gen, device=device).square_().sum(0)
    t = z / torch.sqrt(c / 4.0)
    s = torch.exp(torch.randn((rows, 1), generator=gen, device=device) * 0.5)
    return (t * s).to(dtype)


def torch_generator(device, config, tensor, expert=0):
    import torch
    seed = int(np.random.SeedSequence([config, tensor, expert]).generate_state(1, np.uint64)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed & ((1 << 63) - 1))
    return g


# ---------------------------------------------------------------------------------------
# Routings

def decode_ids(config, step, E, k):
    """k distinct experts for one decode step, uniform without replacement."""
    return rng(config, T_ROUTE, step).choice(E, k, replace=False).astype(np.int32)


def topk_routing(config, T, E, k):
    """Seeded N(0,1) router logits [T, E]; top-k per token (ties to the lower id).
    Returns ids [T*k] in (token, rank) order."""
    logits = rng(config, T_ROUTE).standard_normal((T, E))
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k]
    return order.reshape(-1).astype(np.int32)


def zipf_sorted_routing(config, T, E, k, s=1.1):
    """Zipf(s)-skewed routing for a batch: expert popularity ~ rank^-s over a seeded
    permutation of ranks; each token draws k distinct experts by Gumbel-top-k. Rows (one
    per (token, expert)) are stably sorted by (expert, token).
    Returns row_token [T*k], row_expert [T*k], offsets [E+1] (int32)."""
    g = rng(config, T_ROUTE)
    rank = g.permutation(E) + 1
    logw = -s * np.log(rank.astype(np.float64))
    gumbel = -np.log(-np.log(g.random((T, E))))
    chosen = np.argsort(-(logw[None, :] + gumbel), axis=1, kind="stable")[:, :k]
    tok = np.repeat(np.arange(T), k)
    exp = chosen.reshape(-1)
    order = np.lexsort((tok, exp))
    row_token = tok[order].astype(np.int32)
    row_expert = exp[order].astype(np.int32)
    counts = np.bincount(row_expert, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return row_token, row_expert, offsets


# ---------------------------------------------------------------------------------------
# The five workloads

@dataclass
class Proj:
    name: str
    N: int
    K: int
    levels: int
    group: int
    seed: int


@dataclass
class Config:
    cid: int
    name: str
    E: int
    projs: list = field(default_factory=list)


C1 = Config(1, "single layer 256x512 fp32, 4-bit g64", 1, [Proj("w", 256, 512, 16, 64, 0)])
C2 = Config(2, "dense decode qmv 4096x4096 bf16, 3-bit g128", 1,
            [Proj("w", 4096, 4096, 8, 128, 0)])
C3 = Config(3, "MoE decode gather_qmv: 384 experts, hidden 7168, inter 2048", 384,
            [Proj("gate", 2048, 7168, 4, 64, 0), Proj("up", 2048, 7168, 4, 64, 0),
             Proj("down", 7168, 2048, 16, 64, 1)])
C4 = Config(4, "ternary MoE prefill multi_gather_qmv: 128 experts, hidden 2048, inter 768", 128,
            [Proj("gate", 768, 2048, 3, 16, 0), Proj("up", 768, 2048, 3, 16, 0),
             Proj("down", 2048, 768, 3, 16, 1)])
C5 = Config(5, "batched gather_qmm: 4096 tok x top-8 of 128 experts, hidden 4096, inter 1536",
            128, [Proj("gate", 1536, 4096, 16, 128, 0), Proj("up", 1536, 4096, 16, 128, 0),
                  Proj("down", 4096, 1536, 16, 128, 1)])

CONFIGS = {1: C1, 2: C2, 3: C3, 4: C4, 5: C5}
PROJ_TENSOR = {"w": T_W, "gate": T_GATE, "up": T_UP, "down": T_DOWN}
