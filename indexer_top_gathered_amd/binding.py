"""ctypes binding of libdsa (include/dsa.h), with the same entry-point names.

This layer only marshals arguments: it checks tensor dtypes, shapes and
devices, allocates outputs and workspaces through torch, passes raw device
pointers and the current HIP stream, and turns a non-zero status into an
exception. Every step of the computation runs in the HIP kernels of
libdsa.so; if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_BF16 = 0
DSA_F32 = 1

EXPORTED = (
    "dsa_indexer_score",
    "dsa_topk_workspace_bytes",
    "dsa_topk",
    "dsa_sparse_attend_workspace_bytes",
    "dsa_sparse_attend",
    "dsa_decode_step_workspace_bytes",
    "dsa_decode_step",
    "dsa_topk_ragged",
    "dsa_decode_step_ragged",
    "dsa_indexer_score_mt",
    "dsa_sparse_attend_mt_workspace_bytes",
    "dsa_sparse_attend_mt",
    "dsa_decode_step_mt_workspace_bytes",
    "dsa_decode_step_mt",
    "dsa_indexer_qproj",
    "dsa_decode_step_noalloc",
    "dsa_sparse_attend_sink",
    "dsa_decode_step_sink",
    "dsa_compress",
    "dsa_indexer_topk_workspace_bytes",
    "dsa_indexer_topk",
    "dsa_indexer_topk_chunks",
    "dsa_status_string",
)

# Size of the static workspace of dsa_decode_step_noalloc (DSA_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


class DsaDims(ctypes.Structure):
    """Mirror of dsa_dims_t."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("q_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("scale", ctypes.c_float),
    ]


class DsaError(RuntimeError):
    """A non-zero dsa_status_t."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python indexer_top_gathered_amd/build.py` "
            "(or __graft_entry__.build() at the repository root)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(DsaDims)
    lib.dsa_indexer_score.argtypes = [P, P, P, P, I, I, I, I, P]
    lib.dsa_indexer_score.restype = I
    lib.dsa_topk_workspace_bytes.argtypes = [I, I, I, I]
    lib.dsa_topk_workspace_bytes.restype = S
    lib.dsa_topk.argtypes = [P, I, I, I, I, P, P, I, P, S, P]
    lib.dsa_topk.restype = I
    lib.dsa_sparse_attend_workspace_bytes.argtypes = [D]
    lib.dsa_sparse_attend_workspace_bytes.restype = S
    lib.dsa_sparse_attend.argtypes = [P, P, P, P, P, D, P, S, P]
    lib.dsa_sparse_attend.restype = I
    lib.dsa_decode_step_workspace_bytes.argtypes = [D]
    lib.dsa_decode_step_workspace_bytes.restype = S
    lib.dsa_decode_step.argtypes = [P, P, P, P, P, P, P, P, D, P, S, P]
    lib.dsa_decode_step.restype = I
    lib.dsa_topk_ragged.argtypes = [P, I, I, I, P, I, P, P, I, P, S, P]
    lib.dsa_topk_ragged.restype = I
    lib.dsa_decode_step_ragged.argtypes = [P, P, P, P, P, P, P, P, P, D, P, S, P]
    lib.dsa_decode_step_ragged.restype = I
    lib.dsa_indexer_score_mt.argtypes = [P, P, P, P, I, I, I, I, I, P]
    lib.dsa_indexer_score_mt.restype = I
    lib.dsa_sparse_attend_mt_workspace_bytes.argtypes = [D, I]
    lib.dsa_sparse_attend_mt_workspace_bytes.restype = S
    lib.dsa_sparse_attend_mt.argtypes = [P, P, P, P, P, D, I, P, S, P]
    lib.dsa_sparse_attend_mt.restype = I
    lib.dsa_decode_step_mt_workspace_bytes.argtypes = [D, I]
    lib.dsa_decode_step_mt_workspace_bytes.restype = S
    lib.dsa_decode_step_mt.argtypes = [P, P, P, P, P, P, P, P, P, D, I, P, S, P]
    lib.dsa_decode_step_mt.restype = I
    lib.dsa_indexer_qproj.argtypes = [P, P, P, I, I, I, I, P]
    lib.dsa_indexer_qproj.restype = I
    lib.dsa_decode_step_noalloc.argtypes = [P, P, P, P, P, P, P, P, D, P]
    lib.dsa_decode_step_noalloc.restype = I
    lib.dsa_sparse_attend_sink.argtypes = [P, P, P, P, P, P, D, P, S, P]
    lib.dsa_sparse_attend_sink.restype = I
    lib.dsa_decode_step_sink.argtypes = [P, P, P, P, P, P, P, P, P, D, P, S, P]
    lib.dsa_decode_step_sink.restype = I
    lib.dsa_compress.argtypes = [P, P, P, I, I, I, P]
    lib.dsa_compress.restype = I
    lib.dsa_indexer_topk_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.dsa_indexer_topk_workspace_bytes.restype = S
    lib.dsa_indexer_topk.argtypes = [P, P, P, I, I, I, I, I, P, P, P, S, P]
    lib.dsa_indexer_topk.restype = I
    lib.dsa_indexer_topk_chunks.argtypes = [I, I, I]
    lib.dsa_indexer_topk_chunks.restype = I
    lib.dsa_status_string.argtypes = [I]
    lib.dsa_status_string.restype = ctypes.c_char_p
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.dsa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DsaError(status, where)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on_stream(fn):
    """Run the wrapper with its `stream` argument as torch's current stream,
    so that the outputs and the workspace it allocates belong to the stream
    the kernels run on: the caching allocator then reuses a dropped
    workspace only for work ordered after them on that stream. A raw
    hipStream_t handle is wrapped as an external stream."""
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        st = kwargs.get("stream", args[pos] if len(args) > pos else None)
        if st is None:
            return fn(*args, **kwargs)
        if not isinstance(st, torch.cuda.Stream):
            st = torch.cuda.ExternalStream(int(st))
        if len(args) > pos:
            args = args[:pos] + (st,) + args[pos + 1:]
        else:
            kwargs["stream"] = st
        if st == torch.cuda.current_stream(st.device):
            return fn(*args, **kwargs)
        with torch.cuda.stream(st):
            return fn(*args, **kwargs)
    return wrapper


def _ptr(t: torch.Tensor | None) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(nbytes: int, device, ws: torch.Tensor | None) -> torch.Tensor:
    if ws is None:
        return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if ws.dtype != torch.uint8 or ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous uint8 device tensor")
    return ws


def make_dims(B, N, H_I, D_I, k, W, H_q, D, scale) -> DsaDims:
    return DsaDims(int(B), int(N), int(H_I), int(D_I), int(k), int(W), int(H_q), int(D),
                   float(scale))


# ------------------------------------------------------------------ indexer

@_on_stream
def dsa_indexer_score(q_idx, k_idx, w, scores=None, stream=None):
    """scores[b,j] = sum_h w[b,h] * relu(q_idx[b,h,:] . k_idx[b,j,:]) (float32 [B,N])."""
    B, H, DI = q_idx.shape
    N = k_idx.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, DI))
    _need(w, "w", torch.float32, (B, H))
    if scores is None:
        scores = torch.empty((B, N), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, (B, N))
    _check(LIB.dsa_indexer_score(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(scores), B, N, H, DI,
                                 _stream(stream)), "dsa_indexer_score")
    return scores


@_on_stream
def dsa_indexer_qproj(x, w_q, H_I: int, q_idx=None, stream=None):
    """Indexer query projection: x bf16 [B, d_in], w_q bf16 [H_I*128, d_in]
    -> q_idx bf16 [B, H_I, 128] = x @ w_q^T (fp32 sums, rounded to bf16)."""
    B, d_in = x.shape
    _need(x, "x", torch.bfloat16)
    _need(w_q, "w_q", torch.bfloat16, (H_I * 128, d_in))
    if q_idx is None:
        q_idx = torch.empty((B, H_I, 128), dtype=torch.bfloat16, device=x.device)
    _need(q_idx, "q_idx", torch.bfloat16, (B, H_I, 128))
    _check(LIB.dsa_indexer_qproj(_ptr(x), _ptr(w_q), _ptr(q_idx), B, d_in, int(H_I), 128,
                                 _stream(stream)), "dsa_indexer_qproj")
    return q_idx


@_on_stream
def dsa_indexer_score_mt(q_idx, k_idx, w, scores=None, stream=None):
    """T query tokens per batch row sharing its keys: q_idx bf16 [B,T,H,D_I],
    k_idx [B,N,D_I], w float32 [B,T,H] -> scores float32 [B,T,N]."""
    B, T, H, DI = q_idx.shape
    N = k_idx.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, DI))
    _need(w, "w", torch.float32, (B, T, H))
    if scores is None:
        scores = torch.empty((B, T, N), dtype=torch.float32, device=q_idx.device)
    _need(scores, "scores", torch.float32, (B, T, N))
    _check(LIB.dsa_indexer_score_mt(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(scores), B, T, N, H,
                                    DI, _stream(stream)), "dsa_indexer_score_mt")
    return scores


def dsa_indexer_topk_workspace_bytes(B: int, N: int, H_I: int, k: int,
                                     own_scores: bool = True) -> int:
    return int(LIB.dsa_indexer_topk_workspace_bytes(int(B), int(N), int(H_I), int(k),
                                                    int(bool(own_scores))))


def dsa_indexer_topk_chunks(B: int, N: int, k: int) -> int:
    """Interleaved chunks per row of dsa_indexer_topk (0: unfused kernels)."""
    return int(LIB.dsa_indexer_topk_chunks(int(B), int(N), int(k)))


@_on_stream
def dsa_indexer_topk(q_idx, k_idx, w, k: int, out_idx=None, scores=None, ws=None, stream=None,
                     return_scores: bool = False):
    """Indexer scores and their top-k in one pass: int32 [B, k], the set
    dsa_topk(dsa_indexer_score(q_idx, k_idx, w), k) gives (order unspecified,
    deterministic); with return_scores, also the float32 [B, N] scores."""
    B, H, DI = q_idx.shape
    N = k_idx.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, DI))
    _need(w, "w", torch.float32, (B, H))
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q_idx.device)
    _need(out_idx, "out_idx", torch.int32, (B, k))
    if return_scores and scores is None:
        scores = torch.empty((B, N), dtype=torch.float32, device=q_idx.device)
    if scores is not None:
        _need(scores, "scores", torch.float32, (B, N))
    nbytes = LIB.dsa_indexer_topk_workspace_bytes(B, N, H, int(k), int(scores is None))
    ws = _workspace(nbytes, q_idx.device, ws)
    _check(LIB.dsa_indexer_topk(_ptr(q_idx), _ptr(k_idx), _ptr(w), B, N, H, DI, int(k),
                                _ptr(out_idx), _ptr(scores), _ptr(ws), ws.numel(),
                                _stream(stream)), "dsa_indexer_topk")
    return (out_idx, scores) if scores is not None else out_idx


# ------------------------------------------------------------------ top-k

def dsa_topk_workspace_bytes(B: int, N: int, k: int, dtype=torch.float32) -> int:
    dt = DSA_BF16 if dtype == torch.bfloat16 else DSA_F32
    return int(LIB.dsa_topk_workspace_bytes(int(B), int(N), int(k), dt))


@_on_stream
def dsa_topk(scores, k: int, return_values: bool = False, sorted_index: bool = False,
             out_idx=None, out_val=None, ws=None, stream=None):
    """Indices (int32 [B,k]) of the k largest scores per row, lower index
    first among ties; values are bit copies when return_values."""
    return _topk(scores, None, k, return_values, sorted_index, out_idx, out_val, ws, stream)


@_on_stream
def dsa_topk_ragged(scores, lengths, k: int, return_values: bool = False,
                    sorted_index: bool = False, out_idx=None, out_val=None, ws=None, stream=None):
    """dsa_topk over each row's first lengths[b] scores (lengths: int32 [B]
    on the device); slots past min(k, lengths[b]) hold -1 (values -inf)."""
    return _topk(scores, lengths, k, return_values, sorted_index, out_idx, out_val, ws, stream)


def _topk(scores, lengths, k, return_values, sorted_index, out_idx, out_val, ws, stream):
    if scores.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("scores must be bfloat16 or float32")
    _need(scores, "scores", scores.dtype)
    B, N = scores.shape
    if lengths is not None:
        _need(lengths, "lengths", torch.int32, (B,))
    dt = DSA_BF16 if scores.dtype == torch.bfloat16 else DSA_F32
    if out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    _need(out_idx, "out_idx", torch.int32, (B, k))
    if return_values and out_val is None:
        out_val = torch.empty((B, k), dtype=scores.dtype, device=scores.device)
    if out_val is not None:
        _need(out_val, "out_val", scores.dtype, (B, k))
    nbytes = LIB.dsa_topk_workspace_bytes(B, N, int(k), dt)
    ws = _workspace(nbytes, scores.device, ws)
    if lengths is None:
        _check(LIB.dsa_topk(_ptr(scores), dt, B, N, int(k), _ptr(out_idx), _ptr(out_val),
                            int(bool(sorted_index)), _ptr(ws), ws.numel(), _stream(stream)),
               "dsa_topk")
    else:
        _check(LIB.dsa_topk_ragged(_ptr(scores), dt, B, N, _ptr(lengths), int(k), _ptr(out_idx),
                                   _ptr(out_val), int(bool(sorted_index)), _ptr(ws), ws.numel(),
                                   _stream(stream)), "dsa_topk_ragged")
    return (out_idx, out_val) if out_val is not None else out_idx


# ------------------------------------------------------------------ attention

def dsa_sparse_attend_workspace_bytes(dims: DsaDims) -> int:
    return int(LIB.dsa_sparse_attend_workspace_bytes(ctypes.byref(dims)))


@_on_stream
def dsa_sparse_attend(q, kv_cmp, idx, kv_win, scale: float, out=None, ws=None, stream=None):
    """bf16 [B,H_q,D] = softmax(scale * q R^T) R over R = kv_cmp[idx] ++ kv_win."""
    return _attend(q, kv_cmp, idx, kv_win, None, scale, out, ws, stream)


@_on_stream
def dsa_sparse_attend_sink(q, kv_cmp, idx, kv_win, sink, scale: float, out=None, ws=None,
                           stream=None):
    """dsa_sparse_attend with an attention sink: sink float32 [H_q], one
    logit per query head that joins the softmax normalisation with no value
    vector (-inf: no effect)."""
    return _attend(q, kv_cmp, idx, kv_win, sink, scale, out, ws, stream)


def _attend(q, kv_cmp, idx, kv_win, sink, scale, out, ws, stream):
    B, Hq, D = q.shape
    N = kv_cmp.shape[1]
    k = idx.shape[1]
    W = 0 if kv_win is None else kv_win.shape[1]
    _need(q, "q", torch.bfloat16)
    _need(kv_cmp, "kv_cmp", torch.bfloat16, (B, N, D))
    _need(idx, "idx", torch.int32, (B, k))
    if kv_win is not None:
        _need(kv_win, "kv_win", torch.bfloat16, (B, W, D))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, Hq, D))
    dims = make_dims(B, N, 1, 128, k, W, Hq, D, scale)
    ws = _workspace(LIB.dsa_sparse_attend_workspace_bytes(ctypes.byref(dims)), q.device, ws)
    if sink is None:
        _check(LIB.dsa_sparse_attend(_ptr(q), _ptr(kv_cmp), _ptr(idx),
                                     _ptr(kv_win if W else None), _ptr(out), ctypes.byref(dims),
                                     _ptr(ws), ws.numel(), _stream(stream)), "dsa_sparse_attend")
    else:
        _need(sink, "sink", torch.float32, (Hq,))
        _check(LIB.dsa_sparse_attend_sink(_ptr(q), _ptr(kv_cmp), _ptr(idx),
                                          _ptr(kv_win if W else None), _ptr(sink), _ptr(out),
                                          ctypes.byref(dims), _ptr(ws), ws.numel(),
                                          _stream(stream)), "dsa_sparse_attend_sink")
    return out


@_on_stream
def dsa_sparse_attend_mt(q, kv_cmp, idx, kv_win, scale: float, out=None, ws=None, stream=None):
    """T query tokens per batch row sharing its compressed rows: q bf16
    [B,T,H_q,D], kv_cmp [B,N,D], idx int32 [B,T,k], kv_win [B,T,W,D] or None
    -> bf16 [B,T,H_q,D]."""
    B, T, Hq, D = q.shape
    N = kv_cmp.shape[1]
    k = idx.shape[2]
    W = 0 if kv_win is None else kv_win.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(kv_cmp, "kv_cmp", torch.bfloat16, (B, N, D))
    _need(idx, "idx", torch.int32, (B, T, k))
    if kv_win is not None:
        _need(kv_win, "kv_win", torch.bfloat16, (B, T, W, D))
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, Hq, D))
    dims = make_dims(B, N, 1, 128, k, W, Hq, D, scale)
    ws = _workspace(LIB.dsa_sparse_attend_mt_workspace_bytes(ctypes.byref(dims), T), q.device, ws)
    _check(LIB.dsa_sparse_attend_mt(_ptr(q), _ptr(kv_cmp), _ptr(idx), _ptr(kv_win if W else None),
                                    _ptr(out), ctypes.byref(dims), T, _ptr(ws), ws.numel(),
                                    _stream(stream)), "dsa_sparse_attend_mt")
    return out


# ------------------------------------------------------------------ fused step

def dsa_decode_step_workspace_bytes(dims: DsaDims) -> int:
    return int(LIB.dsa_decode_step_workspace_bytes(ctypes.byref(dims)))


@_on_stream
def dsa_decode_step(q_idx, k_idx, w, q, kv_cmp, kv_win, k: int, scale: float, out=None,
                    out_idx=None, ws=None, stream=None, return_idx: bool = False):
    """Indexer scores -> top-k -> sparse attention in one enqueue sequence."""
    return _step(q_idx, k_idx, w, q, kv_cmp, kv_win, None, k, scale, out, out_idx, ws, stream,
                 return_idx)


@_on_stream
def dsa_decode_step_sink(q_idx, k_idx, w, q, kv_cmp, kv_win, sink, k: int, scale: float,
                         out=None, out_idx=None, ws=None, stream=None, return_idx: bool = False):
    """dsa_decode_step whose attention has a sink (float32 [H_q] logits)."""
    return _step(q_idx, k_idx, w, q, kv_cmp, kv_win, None, k, scale, out, out_idx, ws, stream,
                 return_idx, sink=sink)


@_on_stream
def dsa_decode_step_ragged(q_idx, k_idx, w, q, kv_cmp, kv_win, lengths, k: int, scale: float,
                           out=None, out_idx=None, ws=None, stream=None,
                           return_idx: bool = False):
    """dsa_decode_step over ragged rows (lengths: int32 [B] on the device)."""
    return _step(q_idx, k_idx, w, q, kv_cmp, kv_win, lengths, k, scale, out, out_idx, ws, stream,
                 return_idx)


def _step(q_idx, k_idx, w, q, kv_cmp, kv_win, lengths, k, scale, out, out_idx, ws, stream,
          return_idx, sink=None):
    B, H, DI = q_idx.shape
    N = k_idx.shape[1]
    Hq, D = q.shape[1], q.shape[2]
    W = 0 if kv_win is None else kv_win.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, DI))
    _need(w, "w", torch.float32, (B, H))
    _need(q, "q", torch.bfloat16, (B, Hq, D))
    _need(kv_cmp, "kv_cmp", torch.bfloat16, (B, N, D))
    if kv_win is not None:
        _need(kv_win, "kv_win", torch.bfloat16, (B, W, D))
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, Hq, D))
    if return_idx and out_idx is None:
        out_idx = torch.empty((B, k), dtype=torch.int32, device=q.device)
    if out_idx is not None:
        _need(out_idx, "out_idx", torch.int32, (B, k))
    dims = make_dims(B, N, H, DI, k, W, Hq, D, scale)
    ws = _workspace(LIB.dsa_decode_step_workspace_bytes(ctypes.byref(dims)), q.device, ws)
    if sink is not None:
        _need(sink, "sink", torch.float32, (Hq,))
        _check(LIB.dsa_decode_step_sink(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q), _ptr(kv_cmp),
                                        _ptr(kv_win if W else None), _ptr(sink), _ptr(out),
                                        _ptr(out_idx), ctypes.byref(dims), _ptr(ws), ws.numel(),
                                        _stream(stream)), "dsa_decode_step_sink")
    elif lengths is None:
        _check(LIB.dsa_decode_step(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q), _ptr(kv_cmp),
                                   _ptr(kv_win if W else None), _ptr(out), _ptr(out_idx),
                                   ctypes.byref(dims), _ptr(ws), ws.numel(), _stream(stream)),
               "dsa_decode_step")
    else:
        _need(lengths, "lengths", torch.int32, (B,))
        _check(LIB.dsa_decode_step_ragged(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q),
                                          _ptr(kv_cmp), _ptr(kv_win if W else None),
                                          _ptr(lengths), _ptr(out), _ptr(out_idx),
                                          ctypes.byref(dims), _ptr(ws), ws.numel(),
                                          _stream(stream)), "dsa_decode_step_ragged")
    return (out, out_idx) if out_idx is not None else out


def dsa_decode_step_mt_workspace_bytes(dims: DsaDims, T: int) -> int:
    return int(LIB.dsa_decode_step_mt_workspace_bytes(ctypes.byref(dims), int(T)))


@_on_stream
def dsa_decode_step_mt(q_idx, k_idx, w, q, kv_cmp, kv_win, k: int, scale: float, lengths=None,
                       out=None, out_idx=None, ws=None, stream=None, return_idx: bool = False):
    """The step with T query tokens per batch row sharing its keys: q_idx
    bf16 [B,T,H_I,D_I], k_idx [B,N,D_I], w float32 [B,T,H_I], q [B,T,H_q,D],
    kv_cmp [B,N,D], kv_win [B,T,W,D] or None, lengths int32 [B,T] or None
    -> out bf16 [B,T,H_q,D] (and idx int32 [B,T,k])."""
    B, T, H, DI = q_idx.shape
    N = k_idx.shape[1]
    Hq, D = q.shape[2], q.shape[3]
    W = 0 if kv_win is None else kv_win.shape[2]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, DI))
    _need(w, "w", torch.float32, (B, T, H))
    _need(q, "q", torch.bfloat16, (B, T, Hq, D))
    _need(kv_cmp, "kv_cmp", torch.bfloat16, (B, N, D))
    if kv_win is not None:
        _need(kv_win, "kv_win", torch.bfloat16, (B, T, W, D))
    if lengths is not None:
        _need(lengths, "lengths", torch.int32, (B, T))
    if out is None:
        out = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, (B, T, Hq, D))
    if return_idx and out_idx is None:
        out_idx = torch.empty((B, T, k), dtype=torch.int32, device=q.device)
    if out_idx is not None:
        _need(out_idx, "out_idx", torch.int32, (B, T, k))
    dims = make_dims(B, N, H, DI, k, W, Hq, D, scale)
    ws = _workspace(LIB.dsa_decode_step_mt_workspace_bytes(ctypes.byref(dims), T), q.device, ws)
    _check(LIB.dsa_decode_step_mt(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q), _ptr(kv_cmp),
                                  _ptr(kv_win if W else None), _ptr(lengths), _ptr(out),
                                  _ptr(out_idx), ctypes.byref(dims), T, _ptr(ws), ws.numel(),
                                  _stream(stream)), "dsa_decode_step_mt")
    return (out, out_idx) if out_idx is not None else out


@_on_stream
def dsa_decode_step_noalloc(q_idx, k_idx, w, q, kv_cmp, kv_win, k: int, scale: float, out,
                            out_idx=None, stream=None):
    """dsa_decode_step with the library's static workspace: the C call
    allocates nothing, and this wrapper allocates nothing either (the caller
    passes `out`, and `out_idx` if wanted). Calls that overlap on one GPU
    share that workspace and race."""
    B, H, DI = q_idx.shape
    N = k_idx.shape[1]
    Hq, D = q.shape[1], q.shape[2]
    W = 0 if kv_win is None else kv_win.shape[1]
    _need(q_idx, "q_idx", torch.bfloat16)
    _need(k_idx, "k_idx", torch.bfloat16, (B, N, DI))
    _need(w, "w", torch.float32, (B, H))
    _need(q, "q", torch.bfloat16, (B, Hq, D))
    _need(kv_cmp, "kv_cmp", torch.bfloat16, (B, N, D))
    if kv_win is not None:
        _need(kv_win, "kv_win", torch.bfloat16, (B, W, D))
    _need(out, "out", torch.bfloat16, (B, Hq, D))
    if out_idx is not None:
        _need(out_idx, "out_idx", torch.int32, (B, k))
    dims = make_dims(B, N, H, DI, k, W, Hq, D, scale)
    _check(LIB.dsa_decode_step_noalloc(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q), _ptr(kv_cmp),
                                       _ptr(kv_win if W else None), _ptr(out), _ptr(out_idx),
                                       ctypes.byref(dims), _stream(stream)),
           "dsa_decode_step_noalloc")
    return (out, out_idx) if out_idx is not None else out


@_on_stream
def dsa_compress(x, w_gate, out=None, stream=None):
    """Compressor: x bf16 [B, 4G, D] (raw KV rows, 4 per group), w_gate
    float32 [D] -> bf16 [B, G, D], each group's rows weighted by the softmax
    of their gate scores w_gate . x_i."""
    B, R, D = x.shape
    _need(x, "x", torch.bfloat16)
    if R % 4 != 0:
        raise ValueError("x must hold whole groups of 4 raw rows")
    G = R // 4
    _need(w_gate, "w_gate", torch.float32, (D,))
    if out is None:
        out = torch.empty((B, G, D), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, (B, G, D))
    _check(LIB.dsa_compress(_ptr(x), _ptr(w_gate), _ptr(out), B, G, D, _stream(stream)),
           "dsa_compress")
    return out
