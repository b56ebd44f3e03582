"""Python binding of libtq (include/tq.h): argument marshalling only.

Every step of encode and of the qmv family runs in the HIP kernels of libtq.so; this module
only turns torch tensors into pointers, dtypes and the caller's current HIP stream, and
allocates outputs and workspaces with torch. If libtq.so is missing, every call raises.

The method: turboquant-mlx "How it works" -- "Quantizing a weight, with no data" (rotate,
group RMS, snap to a Lloyd-Max codebook, pack), "The ternary tier (1.58 bits)" and
"Running a quantized layer" (rotate the input, multiply by inline-decoded codes; the MoE
kernels gather_qmv, multi_gather_qmv and gather_qmm).
"""

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "TqError", "QWeight", "lib", "codebook", "words_per_row", "signs", "encode", "fwht",
    "qmv", "gather_qmv", "multi_gather_qmv", "gather_qmm", "workspace_bytes", "dequant",
    "encode_stream", "multi_gather_qmv_static", "ExpertCache", "kv_fetch", "rotate_dense",
    "encode_dense",
    "F32", "BF16", "F16", "X_ROTATED",
]

F32, BF16, F16 = 0, 1, 2
X_ROTATED = 1
OP_QMV, OP_GATHER_QMV, OP_MULTI_GATHER_QMV, OP_GATHER_QMM, OP_ENCODE_DENSE = 1, 2, 3, 4, 5

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class TqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libtq status {status}: {message}")
        self.status = status


class _QWeight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("signs", ctypes.c_void_p),
        ("n_levels", ctypes.c_int32), ("group", ctypes.c_int32),
        ("K", ctypes.c_int64), ("N", ctypes.c_int64), ("E", ctypes.c_int64),
    ]


_lib = None

# (name, restype, argtypes) for every function declared in include/tq.h
_P, _I32, _I64, _U32, _U64, _SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t)
_QW = ctypes.POINTER(_QWeight)
SIGNATURES = [
    ("tq_words_per_row", _I64, [_I64, _I32]),
    ("tq_codebook", ctypes.c_int, [_I32, _P, _P]),
    ("tq_signs", ctypes.c_int, [_U64, _I64, _P, _P]),
    ("tq_encode", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _I32, _I32, _U64, _P, _P, _P]),
    ("tq_fwht", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _U64, _P, ctypes.c_int, _P]),
    ("tq_workspace_bytes", _SZ, [_I32, _QW, _I64, _I64]),
    ("tq_qmv", ctypes.c_int, [_QW, _P, ctypes.c_int, _P, ctypes.c_int, _U32, _P, _SZ, _P]),
    ("tq_gather_qmv", ctypes.c_int,
     [_QW, _P, _I32, _P, ctypes.c_int, _P, ctypes.c_int, _U32, _P, _SZ, _P]),
    ("tq_gather_qmv_pair", ctypes.c_int,
     [_QW, _QW, _P, _I32, _P, ctypes.c_int, _P, ctypes.c_int, _U32, _P]),
    ("tq_multi_gather_qmv", ctypes.c_int,
     [_QW, _P, _I64, _P, ctypes.c_int, _P, ctypes.c_int, _U32, _P, _SZ, _P]),
    ("tq_multi_gather_qmv_pair", ctypes.c_int,
     [_QW, _QW, _P, _I64, _P, ctypes.c_int, _P, ctypes.c_int, _U32, _P, _SZ, _P]),
    ("tq_multi_gather_qmv_static", ctypes.c_int,
     [_QW, _P, _I64, _P, ctypes.c_int, _P, ctypes.c_int, _U32, _P]),
    ("tq_gather_qmm", ctypes.c_int,
     [_QW, _P, ctypes.c_int, _I64, _P, _P, _I64, _P, ctypes.c_int, _U32, _P, _SZ, _P]),
    ("tq_gather_qmm_pair", ctypes.c_int,
     [_QW, _QW, _P, ctypes.c_int, _I64, _P, _P, _I64, _P, ctypes.c_int, _U32, _P, _SZ, _P]),
    ("tq_dequant", ctypes.c_int, [_QW, _P, _I64, _P, ctypes.c_int, _P]),
    ("tq_encode_stream", ctypes.c_int,
     [_P, ctypes.c_int, _I64, _I64, _I32, _I32, _U64, _P, _P, _P, _SZ, _P, _P]),
    ("tq_kv_fetch", ctypes.c_int, [_QW, _P, ctypes.c_int, _P]),
    ("tq_rotate_dense", ctypes.c_int, [_P, ctypes.c_int, _I64, _I64, _P, _P, ctypes.c_int, _P]),
    ("tq_encode_dense", ctypes.c_int,
     [_P, ctypes.c_int, _I64, _I64, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    ("tq_expert_cache_bytes", _SZ, [_I32, _I64]),
    ("tq_expert_cache_init", ctypes.c_int, [_P, _SZ, _I32, _I64]),
    ("tq_expert_cache_fetch", ctypes.c_int, [_P, _QW, _QW, _P, _I32, _P, _P, _P, _P, _P]),
    ("tq_expert_cache_stats", ctypes.c_int, [_P, _P, _P]),
    ("tq_last_error", ctypes.c_char_p, []),
]


def lib():
    """The loaded libtq.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m rotation_lloyd_max_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status):
    if status != 0:
        raise TqError(status, lib().tq_last_error().decode())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dt(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _out(out, shape, dtype, device):
    """A new output tensor, or the caller's out= once it is known to hold exactly the
    elements the call writes (the library writes through the pointer, so a smaller or
    strided buffer would be written past its end)."""
    shape = (shape,) if isinstance(shape, int) else tuple(shape)
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    n = 1
    for d in shape:
        n *= int(d)
    if out.numel() != n or not out.is_contiguous() or out.device != torch.device(device):
        raise ValueError(f"out= must be a contiguous tensor of {n} elements {tuple(shape)} on "
                         f"{device}, got {tuple(out.shape)} on {out.device}")
    return out


def words_per_row(K, levels):
    return int(lib().tq_words_per_row(K, levels))


def codebook(levels):
    """(centroids, thresholds) as float32 numpy arrays, from the library."""
    c = np.zeros(256, dtype=np.float32)
    t = np.zeros(255, dtype=np.float32)
    _check(lib().tq_codebook(levels, c.ctypes.data, t.ctypes.data))
    return c[:levels].copy(), t[:levels - 1].copy()


def signs(seed, K, device="cuda"):
    """Rotation sign bits for (seed, K) as an int32 tensor of ceil(K/32) words."""
    out = torch.empty((K + 31) // 32, dtype=torch.int32, device=device)
    _check(lib().tq_signs(seed, K, _ptr(out), _stream()))
    return out


@dataclass
class QWeight:
    """Packed weight of E experts of N x K: codes int32 [E, N, wpr] (uint32 bit patterns),
    scales float16 [E, N, K/group], signs int32 [ceil(K/32)] = signs(seed, K). The seed is
    the record of the rotation; the library reads only the sign bits made from it."""
    codes: torch.Tensor
    scales: torch.Tensor
    signs: torch.Tensor
    levels: int
    group: int
    K: int
    N: int
    E: int
    seed: int

    def desc(self):
        sg = self.signs.data_ptr() if self.signs.numel() else 0
        return _QWeight(self.codes.data_ptr(), self.scales.data_ptr(), sg,
                        self.levels, self.group, self.K, self.N, self.E)

    def expert(self, e):
        """View of expert e as a dense (E = 1) weight."""
        return QWeight(self.codes[e:e + 1], self.scales[e:e + 1], self.signs, self.levels,
                       self.group, self.K, self.N, 1, self.seed)


def _check_out(out, E, N, K, levels, group, seed, device):
    """An out= weight must be exactly the one the call writes: the library writes E*N rows
    of codes and scales through its pointers."""
    wpr = words_per_row(K, levels)
    want = {"levels": levels, "group": group, "K": K, "N": N, "E": E, "seed": seed}
    got = {k: getattr(out, k) for k in want}
    if got != want:
        raise ValueError(f"out= describes {got}, the call writes {want}")
    for name, t, shape, dt in (("codes", out.codes, (E, N, wpr), torch.int32),
                               ("scales", out.scales, (E, N, K // group), torch.float16)):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"out.{name} must be a contiguous {dt} tensor of shape {shape}")
        if t.device != torch.device(device):
            raise ValueError(f"out.{name} is on {t.device}, the call writes on {device}")


def encode(W, levels, group, seed, out=None):
    """Quantize W ([N, K] or [E, N, K], float32/bfloat16/float16 on the GPU)."""
    if W.dim() == 2:
        W = W.unsqueeze(0)
    W = W.contiguous()
    E, N, K = W.shape
    wpr = words_per_row(K, levels)
    if out is None:
        codes = torch.empty((E, N, wpr), dtype=torch.int32, device=W.device)
        scales = torch.empty((E, N, K // group), dtype=torch.float16, device=W.device)
        sg = signs(seed, K, W.device)
    else:
        _check_out(out, E, N, K, levels, group, seed, W.device)
        codes, scales, sg = out.codes, out.scales, out.signs
    with torch.cuda.device(W.device):
        _check(lib().tq_encode(_ptr(W), _dt(W), E * N, K, levels, group, seed, _ptr(codes),
                               _ptr(scales), _stream(W.device)))
    return QWeight(codes, scales, sg, levels, group, K, N, E, seed)


_copy_streams = {}


def _copy_stream(device):
    """One copy stream per device (default priority), created on first use."""
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _copy_streams:
        _copy_streams[idx] = torch.cuda.Stream(device=idx)
    return _copy_streams[idx]


def encode_stream(W_host, levels, group, seed, device="cuda", staging_bytes=64 << 20,
                  out=None, copy_stream=None):
    """encode() of a weight held in host memory ([N, K] or [E, N, K] contiguous CPU tensor,
    pinned for overlap), streamed to the device through a staging buffer of staging_bytes;
    the same bytes as encode() of the whole weight on the device. The copies read W_host
    after this returns: keep it alive and unchanged until the current stream has passed
    this call. copy_stream: a torch.cuda.Stream for the copies (default: one kept per
    device), or the current stream for no overlap."""
    if W_host.device.type != "cpu":
        raise ValueError("encode_stream takes a host (CPU) tensor")
    if not W_host.is_contiguous():
        raise ValueError("encode_stream needs a contiguous W_host (the copies are asynchronous)")
    if W_host.dim() == 2:
        W_host = W_host.unsqueeze(0)
    E, N, K = W_host.shape
    device = torch.device(device)
    if device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    wpr = words_per_row(K, levels)
    if out is None:
        codes = torch.empty((E, N, wpr), dtype=torch.int32, device=device)
        scales = torch.empty((E, N, K // group), dtype=torch.float16, device=device)
        sg = signs(seed, K, device)
    else:
        _check_out(out, E, N, K, levels, group, seed, device)
        codes, scales, sg = out.codes, out.scales, out.signs
    staging = _workspace(staging_bytes, device)
    cs = copy_stream if copy_stream is not None else _copy_stream(device)
    # the library orders the first copies after the work already on the encode stream
    # (which may still use the staging memory torch hands out again)
    with torch.cuda.device(device):
        _check(lib().tq_encode_stream(_ptr(W_host), _dt(W_host), E * N, K, levels, group,
                                      seed, _ptr(codes), _ptr(scales), _ptr(staging),
                                      staging_bytes, _stream(device),
                                      ctypes.c_void_p(cs.cuda_stream)))
    # the copy stream wrote the staging buffer; keep it alive for that stream too
    staging.record_stream(cs)
    return QWeight(codes, scales, sg, levels, group, K, N, E, seed)


def fwht(x, seed, out_dtype=torch.float32):
    """R x for each row of x ([rows, K])."""
    x = x.contiguous()
    K = x.shape[-1]
    rows = x.numel() // K
    out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    _check(lib().tq_fwht(_ptr(x), _dt(x), rows, K, seed, _ptr(out), _dt(out), _stream()))
    return out


def workspace_bytes(op, qw, count=0, T=0):
    d = qw.desc()
    n = lib().tq_workspace_bytes(op, ctypes.byref(d), count, T)
    if n == ctypes.c_size_t(-1).value:
        raise TqError(-1, lib().tq_last_error().decode())
    return int(n)


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    # int64 storage keeps torch's (256-byte aligned) allocation; size in 8-byte units
    return torch.empty((nbytes + 7) // 8, dtype=torch.int64, device=device)


def qmv(qw, x, out_dtype=torch.float32, rotated=False, out=None):
    x = x.contiguous()
    y = _out(out, qw.N, out_dtype, x.device)
    d = qw.desc()
    _check(lib().tq_qmv(ctypes.byref(d), _ptr(x), _dt(x), _ptr(y), _dt(y),
                        X_ROTATED if rotated else 0, None, 0, _stream()))
    return y


def rotate_dense(x, R, out_dtype=torch.float32, out=None):
    """R x for each row of x ([rows, K]); R a [K, K] float32 rotation on the same device."""
    x = x.contiguous()
    K = x.shape[-1]
    rows = x.numel() // K
    if R.dtype != torch.float32 or tuple(R.shape) != (K, K):
        raise ValueError("R must be a float32 [K, K] tensor")
    R = R.contiguous()
    o = _out(out, x.shape, out_dtype, x.device)
    with torch.cuda.device(x.device):
        _check(lib().tq_rotate_dense(_ptr(x), _dt(x), rows, K, _ptr(R), _ptr(o), _dt(o),
                                     _stream(x.device)))
    return o


def encode_dense(W, R, levels, group, ws_bytes=256 << 20, out=None):
    """encode() with the dense rotation R ([K, K] float32) in place of the Hadamard one. The
    returned QWeight has no sign bits (signs is an empty tensor): run its layers on inputs
    rotated with rotate_dense(x, R) and rotated=True. seed is recorded as -1."""
    if W.dim() == 2:
        W = W.unsqueeze(0)
    W = W.contiguous()
    E, N, K = W.shape
    if R.dtype != torch.float32 or tuple(R.shape) != (K, K):
        raise ValueError("R must be a float32 [K, K] tensor")
    R = R.contiguous()
    wpr = words_per_row(K, levels)
    if out is None:
        codes = torch.empty((E, N, wpr), dtype=torch.int32, device=W.device)
        scales = torch.empty((E, N, K // group), dtype=torch.float16, device=W.device)
    else:
        codes, scales = out.codes, out.scales
    nbytes = min(ws_bytes, E * N * K * 8)
    nbytes = max(nbytes, K * 8)
    ws = _workspace(nbytes, W.device)
    with torch.cuda.device(W.device):
        _check(lib().tq_encode_dense(_ptr(W), _dt(W), E * N, K, _ptr(R), levels, group,
                                     _ptr(codes), _ptr(scales), _ptr(ws), nbytes,
                                     _stream(W.device)))
    empty = torch.empty(0, dtype=torch.int32, device=W.device)
    return QWeight(codes, scales, empty, levels, group, K, N, E, -1)


def kv_fetch(qw, out_dtype=torch.bfloat16, out=None):
    """Every row of a compressed KV cache (a QWeight of E x N rows of head_dim K, typically
    from encode(x, 256 or 8, group, seed)) dequantized and rotated back: [E, N, K]."""
    o = _out(out, (qw.E, qw.N, qw.K), out_dtype, qw.codes.device)
    d = qw.desc()
    with torch.cuda.device(qw.codes.device):
        _check(lib().tq_kv_fetch(ctypes.byref(d), _ptr(o), _dt(o), _stream(qw.codes.device)))
    return o


def dequant(qw, ids=None, out_dtype=torch.bfloat16, out=None):
    """Decoded weights [n][N][K] of experts ids (all E when None), in the rotated basis."""
    if ids is not None:
        ids = ids.to(torch.int32).contiguous()
        n = ids.numel()
    else:
        n = qw.E
    dev = qw.codes.device
    w = _out(out, (n, qw.N, qw.K), out_dtype, dev)
    d = qw.desc()
    _check(lib().tq_dequant(ctypes.byref(d), _ptr(ids) if ids is not None else None, n,
                            _ptr(w), _dt(w), _stream()))
    return w


def gather_qmv(qw, ids, x, out_dtype=torch.float32, rotated=False, out=None):
    x = x.contiguous()
    ids = ids.to(torch.int32).contiguous()
    n = ids.numel()
    y = _out(out, (n, qw.N), out_dtype, x.device)
    d = qw.desc()
    _check(lib().tq_gather_qmv(ctypes.byref(d), _ptr(ids), n, _ptr(x), _dt(x), _ptr(y), _dt(y),
                               X_ROTATED if rotated else 0, None, 0, _stream()))
    return y


def gather_qmv_pair(qw1, qw2, ids, x, out_dtype=torch.float32, rotated=False, out=None):
    """gather_qmv of two weights sharing the routed ids and the input (gate and up of a MoE
    layer) in one launch: [2n, N], rows n.. from qw2. The weights must be rotated alike
    (same seed and K); the library then reads one sign array, qw1's."""
    if qw1.seed != qw2.seed or qw1.K != qw2.K:
        raise ValueError("gather_qmv_pair: the two weights must share seed and K")
    x = x.contiguous()
    ids = ids.to(torch.int32).contiguous()
    n = ids.numel()
    y = _out(out, (2 * n, qw1.N), out_dtype, x.device)
    d1 = qw1.desc()
    d2 = qw2.desc()
    d2.signs = d1.signs
    _check(lib().tq_gather_qmv_pair(ctypes.byref(d1), ctypes.byref(d2), _ptr(ids), n, _ptr(x),
                                    _dt(x), _ptr(y), _dt(y), X_ROTATED if rotated else 0,
                                    _stream()))
    return y


def multi_gather_qmv(qw, ids, X, out_dtype=torch.float32, rotated=False, out=None, ws=None):
    X = X.contiguous()
    ids = ids.to(torch.int32).contiguous()
    P = ids.numel()
    y = _out(out, (P, qw.N), out_dtype, X.device)
    nbytes = workspace_bytes(OP_MULTI_GATHER_QMV, qw, P)
    if ws is None:
        ws = _workspace(nbytes, X.device)
    d = qw.desc()
    _check(lib().tq_multi_gather_qmv(ctypes.byref(d), _ptr(ids), P, _ptr(X), _dt(X), _ptr(y),
                                     _dt(y), X_ROTATED if rotated else 0, _ptr(ws), nbytes,
                                     _stream()))
    return y


def multi_gather_qmv_pair(qw1, qw2, ids, X, out_dtype=torch.float32, rotated=False, out=None,
                          ws=None):
    """multi_gather_qmv of two weights over the same (input, expert) pairs (gate and up of a
    MoE layer) in one call: [2P, N], rows P.. from qw2. The weights must be rotated alike
    (same seed and K); the library then reads one sign array, qw1's."""
    if qw1.seed != qw2.seed or qw1.K != qw2.K:
        raise ValueError("multi_gather_qmv_pair: the two weights must share seed and K")
    X = X.contiguous()
    ids = ids.to(torch.int32).contiguous()
    P = ids.numel()
    y = _out(out, (2 * P, qw1.N), out_dtype, X.device)
    nbytes = workspace_bytes(OP_MULTI_GATHER_QMV, qw1, P)
    if ws is None:
        ws = _workspace(nbytes, X.device)
    d1 = qw1.desc()
    d2 = qw2.desc()
    d2.signs = d1.signs
    _check(lib().tq_multi_gather_qmv_pair(ctypes.byref(d1), ctypes.byref(d2), _ptr(ids), P,
                                          _ptr(X), _dt(X), _ptr(y), _dt(y),
                                          X_ROTATED if rotated else 0, _ptr(ws), nbytes,
                                          _stream()))
    return y


def multi_gather_qmv_static(qw, ids, X, out_dtype=torch.float32, rotated=False, out=None):
    """multi_gather_qmv with the library's fixed per-GPU workspace (no allocation in the
    library; at most 8 MiB of workspace, see tq.h)."""
    X = X.contiguous()
    ids = ids.to(torch.int32).contiguous()
    P = ids.numel()
    y = _out(out, (P, qw.N), out_dtype, X.device)
    d = qw.desc()
    with torch.cuda.device(X.device):
        _check(lib().tq_multi_gather_qmv_static(ctypes.byref(d), _ptr(ids), P, _ptr(X), _dt(X),
                                                _ptr(y), _dt(y), X_ROTATED if rotated else 0,
                                                _stream(X.device)))
    return y


def gather_qmm(qw, X, row_token, offsets, out_dtype=torch.float32, rotated=False, out=None,
               ws=None):
    X = X.contiguous()
    row_token = row_token.to(torch.int32).contiguous()
    offsets = offsets.to(torch.int32).contiguous()
    T = X.shape[0]
    M = row_token.numel()
    y = _out(out, (M, qw.N), out_dtype, X.device)
    nbytes = workspace_bytes(OP_GATHER_QMM, qw, M, T)
    if ws is None:
        ws = _workspace(nbytes, X.device)
    d = qw.desc()
    _check(lib().tq_gather_qmm(ctypes.byref(d), _ptr(X), _dt(X), T, _ptr(row_token),
                               _ptr(offsets), M, _ptr(y), _dt(y),
                               X_ROTATED if rotated else 0, _ptr(ws), nbytes, _stream()))
    return y


def gather_qmm_pair(qw1, qw2, X, row_token, offsets, out_dtype=torch.float32, rotated=False,
                    out=None, ws=None):
    """gather_qmm of two weights over the same sorted rows (gate and up of a MoE layer):
    [2M, N], rows M.. from qw2; the rows are rotated and the tiles scheduled once. The
    weights must be rotated alike (same seed and K); the library then reads qw1's signs."""
    if qw1.seed != qw2.seed or qw1.K != qw2.K:
        raise ValueError("gather_qmm_pair: the two weights must share seed and K")
    X = X.contiguous()
    row_token = row_token.to(torch.int32).contiguous()
    offsets = offsets.to(torch.int32).contiguous()
    T = X.shape[0]
    M = row_token.numel()
    y = _out(out, (2 * M, qw1.N), out_dtype, X.device)
    nbytes = workspace_bytes(OP_GATHER_QMM, qw1, M, T)
    if ws is None:
        ws = _workspace(nbytes, X.device)
    d1 = qw1.desc()
    d2 = qw2.desc()
    d2.signs = d1.signs
    _check(lib().tq_gather_qmm_pair(ctypes.byref(d1), ctypes.byref(d2), _ptr(X), _dt(X), T,
                                    _ptr(row_token), _ptr(offsets), M, _ptr(y), _dt(y),
                                    X_ROTATED if rotated else 0, _ptr(ws), nbytes, _stream()))
    return y


class ExpertCache:
    """Expert streaming: `host` is a QWeight whose codes and scales are CPU tensors (pinned
    for asynchronous copies) and whose signs are on the device; `slots` experts at a time
    live in a device pool, replaced least recently used first. fetch(ids) makes ids resident
    and returns their slot numbers on the device; gather_qmv / multi_gather_qmv run the
    layer on the pool with results bit-identical to the all-resident weight."""

    def __init__(self, host, slots, device="cuda", copy_stream=None):
        if host.codes.device.type != "cpu" or host.scales.device.type != "cpu":
            raise ValueError("ExpertCache takes a weight whose codes and scales are in host memory")
        self.host = host
        self.device = torch.device(device)
        self.copy_stream = copy_stream
        nbytes = lib().tq_expert_cache_bytes(slots, host.E)
        if nbytes == ctypes.c_size_t(-1).value:
            raise ValueError("slots and E must be in [1, 8192]")
        self.state = np.zeros((nbytes + 7) // 8, dtype=np.uint64)
        _check(lib().tq_expert_cache_init(self.state.ctypes.data, self.state.nbytes, slots, host.E))
        self.pool = QWeight(
            torch.empty((slots,) + tuple(host.codes.shape[1:]), dtype=torch.int32, device=self.device),
            torch.empty((slots,) + tuple(host.scales.shape[1:]), dtype=torch.float16, device=self.device),
            host.signs, host.levels, host.group, host.K, host.N, slots, host.seed)
        self.slot_ids = torch.empty(512, dtype=torch.int32, device=self.device)

    def fetch(self, ids):
        """Make experts `ids` (host ints) resident; returns (slot ids on the device, number
        of experts copied)."""
        ids = np.ascontiguousarray(np.asarray(ids, dtype=np.int32).reshape(-1))
        n = ids.size
        copied = ctypes.c_int32(0)
        hd, pd = self.host.desc(), self.pool.desc()
        cs = ctypes.c_void_p(self.copy_stream.cuda_stream) if self.copy_stream is not None else None
        with torch.cuda.device(self.device):
            _check(lib().tq_expert_cache_fetch(self.state.ctypes.data, ctypes.byref(hd),
                                               ctypes.byref(pd), ids.ctypes.data, n,
                                               _ptr(self.slot_ids), None, ctypes.byref(copied),
                                               _stream(self.device), cs))
        return self.slot_ids[:n], int(copied.value)

    def stats(self):
        h, m = ctypes.c_int64(0), ctypes.c_int64(0)
        _check(lib().tq_expert_cache_stats(self.state.ctypes.data, ctypes.byref(h), ctypes.byref(m)))
        return int(h.value), int(m.value)

    def gather_qmv(self, ids, x, **kw):
        sid, _ = self.fetch(ids)
        return gather_qmv(self.pool, sid, x, **kw)

    def multi_gather_qmv(self, ids, X, **kw):
        sid, _ = self.fetch(ids)
        return multi_gather_qmv(self.pool, sid, X, **kw)
