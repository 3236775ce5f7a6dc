"""CPU oracle for the sparse-attention decode step.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The GPU library never imports,
links or calls it, and it imports nothing from the GPU library.

``oracle.c`` holds the plain double-precision definitions (indexer score,
top-k by a full sort, softmax attention, the composed step); this module
compiles it with gcc into ``liboracle.so`` on first use and exposes numpy
wrappers. ``brute.py`` holds pure-Python O(N^2) and closed-form checks for tiny
inputs that pin the C code.

Sources: "feat: Add DeepSeek-V4 CSA attention kernels" (aws-neuron
nki-library pull request 13), section "How the algorithm works", steps 2-4;
"DeepSelect" project page (deepseek-ai/DeepSelect), algorithm and scenario
paragraphs.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

BF16 = 0
F32 = 1


def compile_source(src: str, dst: str) -> str:
    """Compile a C oracle source with gcc (-O2, OpenMP, no fast math, no FMA
    contraction) into the shared library dst."""
    tmp = dst + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, dst)
    return dst


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    return compile_source(_SRC, _LIB_PATH)


def source_path() -> str:
    """Path of oracle.c."""
    return _SRC


@contextlib.contextmanager
def using_library(path: str):
    """Route every oracle call through the library at path for the duration
    (a build of a deliberately altered copy of oracle.c: the tests use it to
    show that the pins catch planted mistakes)."""
    global _lib
    lib = _configure(ctypes.CDLL(path))
    with _lock:
        saved = _lib
        _lib = lib
    try:
        yield
    finally:
        with _lock:
            _lib = saved


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = _configure(ctypes.CDLL(build(force=False)))
    return _lib


def _configure(lib):
    """Argument and result types of every oracle entry point."""
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.oracle_bf16_decode.argtypes = [P, P, ctypes.c_int64]
    lib.oracle_bf16_decode.restype = None
    lib.oracle_indexer.argtypes = [P, P, P, P, I, I, I, I]
    lib.oracle_indexer.restype = None
    lib.oracle_topk.argtypes = [P, I, I, I, I, P, I]
    lib.oracle_topk.restype = I
    lib.oracle_attend.argtypes = [P, P, P, P, P, I, I, I, I, I, I, ctypes.c_double]
    lib.oracle_attend.restype = I
    lib.oracle_step.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                ctypes.c_double]
    lib.oracle_step.restype = I
    lib.oracle_topk_ragged.argtypes = [P, I, I, I, P, I, P, I]
    lib.oracle_topk_ragged.restype = I
    lib.oracle_step_ragged.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                       I, ctypes.c_double]
    lib.oracle_step_ragged.restype = I
    lib.oracle_indexer_mt.argtypes = [P, P, P, P, I, I, I, I, I]
    lib.oracle_indexer_mt.restype = None
    lib.oracle_attend_mt.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I,
                                     ctypes.c_double]
    lib.oracle_attend_mt.restype = I
    lib.oracle_step_mt.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I,
                                   I, ctypes.c_double]
    lib.oracle_step_mt.restype = I
    lib.oracle_qproj.argtypes = [P, P, P, I, I, I]
    lib.oracle_qproj.restype = None
    lib.oracle_attend_sink.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, ctypes.c_double]
    lib.oracle_attend_sink.restype = I
    lib.oracle_compress.argtypes = [P, P, P, I, I, I]
    lib.oracle_compress.restype = None
    lib.oracle_set_threads.argtypes = [I]
    lib.oracle_set_threads.restype = None
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = I
    return lib


def set_threads(n: int) -> None:
    """Set the OpenMP thread count used by the C oracle (it only splits rows)."""
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    """Threads the C oracle's parallel loops will use."""
    return int(_load().oracle_max_threads())


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    _load().oracle_bf16_decode(_ptr(bits), _ptr(out), bits.size)
    return out


def indexer(q_idx: np.ndarray, k_idx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Indexer scores. q_idx uint16(bf16) [B,H,D], k_idx uint16 [B,N,D],
    w float32 [B,H] -> float32 [B,N]."""
    q_idx = _c(q_idx, np.uint16)
    k_idx = _c(k_idx, np.uint16)
    w = _c(w, np.float32)
    B, H, D = q_idx.shape
    N = k_idx.shape[1]
    assert k_idx.shape == (B, N, D) and w.shape == (B, H)
    s = np.empty((B, N), np.float32)
    _load().oracle_indexer(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(s), B, N, H, D)
    return s


def topk(scores: np.ndarray, k: int, index_order: bool = False) -> np.ndarray:
    """Top-k indices per row. scores: float32 [B,N] or uint16 bf16 bits [B,N].
    Order: value desc then index asc, or ascending index if index_order."""
    scores = np.ascontiguousarray(scores)
    if scores.dtype == np.uint16:
        dt = BF16
    elif scores.dtype == np.float32:
        dt = F32
    else:
        raise TypeError("scores must be float32 or uint16 (bf16 bits)")
    B, N = scores.shape
    idx = np.empty((B, k), np.int32)
    rc = _load().oracle_topk(_ptr(scores), dt, B, N, int(k), _ptr(idx), int(bool(index_order)))
    if rc != 0:
        raise ValueError("oracle_topk: invalid arguments")
    return idx


def topk_ragged(scores: np.ndarray, lengths: np.ndarray, k: int,
                index_order: bool = False) -> np.ndarray:
    """Top-k over the first lengths[b] scores of each row; slots past
    min(k, lengths[b]) hold -1. Same dtypes and orders as topk."""
    scores = np.ascontiguousarray(scores)
    if scores.dtype == np.uint16:
        dt = BF16
    elif scores.dtype == np.float32:
        dt = F32
    else:
        raise TypeError("scores must be float32 or uint16 (bf16 bits)")
    B, N = scores.shape
    lengths = _c(lengths, np.int32)
    assert lengths.shape == (B,)
    idx = np.empty((B, k), np.int32)
    rc = _load().oracle_topk_ragged(_ptr(scores), dt, B, N, _ptr(lengths), int(k), _ptr(idx),
                                    int(bool(index_order)))
    if rc != 0:
        raise ValueError("oracle_topk_ragged: invalid arguments")
    return idx


def attend(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, win: np.ndarray | None,
           scale: float, sink: np.ndarray | None = None) -> np.ndarray:
    """Sparse attention. q uint16 [B,Hq,D], kv uint16 [B,N,D], idx int32 [B,k]
    (-1: an empty slot, no row), win uint16 [B,W,D] or None -> float64
    [B,Hq,D]; a batch row with no rows at all gets zeros. sink: float64
    [Hq] (finite or -inf), one logit per query head that joins the softmax
    normalisation with no value vector, or None for none."""
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    idx = _c(idx, np.int32)
    B, Hq, D = q.shape
    N = kv.shape[1]
    k = idx.shape[1]
    if win is None or win.size == 0:
        W = 0
        win = np.zeros((1,), np.uint16)
    else:
        win = _c(win, np.uint16)
        W = win.shape[1]
        assert win.shape == (B, W, D)
    out = np.empty((B, Hq, D), np.float64)
    if sink is None:
        rc = _load().oracle_attend(_ptr(q), _ptr(kv), _ptr(idx), _ptr(win), _ptr(out),
                                   B, N, k, W, Hq, D, float(scale))
    else:
        sink = _c(sink, np.float64)
        assert sink.shape == (Hq,)
        rc = _load().oracle_attend_sink(_ptr(q), _ptr(kv), _ptr(idx), _ptr(win), _ptr(sink),
                                        _ptr(out), B, N, k, W, Hq, D, float(scale))
    if rc != 0:
        raise ValueError("oracle_attend: index out of range or empty row set")
    return out


def step(q_idx, k_idx, w, q, kv, win, k: int, scale: float):
    """Whole decode step; returns (scores float32 [B,N], idx int32 [B,k] in
    value-desc order, out float64 [B,Hq,D])."""
    q_idx = _c(q_idx, np.uint16)
    k_idx = _c(k_idx, np.uint16)
    w = _c(w, np.float32)
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    B, H, DI = q_idx.shape
    N = k_idx.shape[1]
    Hq, D = q.shape[1], q.shape[2]
    if win is None or win.size == 0:
        W = 0
        win = np.zeros((1,), np.uint16)
    else:
        win = _c(win, np.uint16)
        W = win.shape[1]
    scores = np.empty((B, N), np.float32)
    idx = np.empty((B, k), np.int32)
    out = np.empty((B, Hq, D), np.float64)
    rc = _load().oracle_step(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q), _ptr(kv), _ptr(win),
                             _ptr(scores), _ptr(idx), _ptr(out), B, N, H, DI, int(k), W, Hq, D,
                             float(scale))
    if rc != 0:
        raise ValueError("oracle_step: invalid arguments")
    return scores, idx, out


def step_ragged(q_idx, k_idx, w, q, kv, win, lengths, k: int, scale: float):
    """The step over ragged rows (row b's top-k looks at its first lengths[b]
    scores; empty slots, -1, take no part in attention). Returns (scores,
    idx, out) as step does."""
    q_idx = _c(q_idx, np.uint16)
    k_idx = _c(k_idx, np.uint16)
    w = _c(w, np.float32)
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    lengths = _c(lengths, np.int32)
    B, H, DI = q_idx.shape
    N = k_idx.shape[1]
    Hq, D = q.shape[1], q.shape[2]
    if win is None or win.size == 0:
        W = 0
        win = np.zeros((1,), np.uint16)
    else:
        win = _c(win, np.uint16)
        W = win.shape[1]
    scores = np.empty((B, N), np.float32)
    idx = np.empty((B, k), np.int32)
    out = np.empty((B, Hq, D), np.float64)
    rc = _load().oracle_step_ragged(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q), _ptr(kv),
                                    _ptr(win), _ptr(lengths), _ptr(scores), _ptr(idx), _ptr(out),
                                    B, N, H, DI, int(k), W, Hq, D, float(scale))
    if rc != 0:
        raise ValueError("oracle_step_ragged: invalid arguments")
    return scores, idx, out


def _window(win, lead: tuple, D: int):
    """(array, W) for a window argument that may be None or empty."""
    if win is None or win.size == 0:
        return np.zeros((1,), np.uint16), 0
    win = _c(win, np.uint16)
    W = win.shape[len(lead)]
    assert win.shape == lead + (W, D)
    return win, W


def indexer_mt(q_idx: np.ndarray, k_idx: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Indexer scores with T query tokens per batch row sharing its keys.
    q_idx uint16 [B,T,H,D], k_idx uint16 [B,N,D], w float32 [B,T,H] ->
    float32 [B,T,N]."""
    q_idx = _c(q_idx, np.uint16)
    k_idx = _c(k_idx, np.uint16)
    w = _c(w, np.float32)
    B, T, H, D = q_idx.shape
    N = k_idx.shape[1]
    assert k_idx.shape == (B, N, D) and w.shape == (B, T, H)
    s = np.empty((B, T, N), np.float32)
    _load().oracle_indexer_mt(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(s), B, T, N, H, D)
    return s


def attend_mt(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, win, scale: float) -> np.ndarray:
    """Sparse attention with T query tokens per batch row sharing its
    compressed rows. q uint16 [B,T,Hq,D], kv uint16 [B,N,D], idx int32
    [B,T,k] (-1: empty slot), win uint16 [B,T,W,D] or None -> float64
    [B,T,Hq,D]."""
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    idx = _c(idx, np.int32)
    B, T, Hq, D = q.shape
    N = kv.shape[1]
    k = idx.shape[2]
    assert kv.shape == (B, N, D) and idx.shape == (B, T, k)
    win, W = _window(win, (B, T), D)
    out = np.empty((B, T, Hq, D), np.float64)
    rc = _load().oracle_attend_mt(_ptr(q), _ptr(kv), _ptr(idx), _ptr(win), _ptr(out),
                                  B, T, N, k, W, Hq, D, float(scale))
    if rc != 0:
        raise ValueError("oracle_attend_mt: index out of range or empty row set")
    return out


def step_mt(q_idx, k_idx, w, q, kv, win, lengths, k: int, scale: float):
    """The step with T query tokens per batch row (shapes as indexer_mt and
    attend_mt; lengths int32 [B,T] or None for full rows). Returns (scores
    float32 [B,T,N], idx int32 [B,T,k] in value-desc order, out float64
    [B,T,Hq,D])."""
    q_idx = _c(q_idx, np.uint16)
    k_idx = _c(k_idx, np.uint16)
    w = _c(w, np.float32)
    q = _c(q, np.uint16)
    kv = _c(kv, np.uint16)
    B, T, H, DI = q_idx.shape
    N = k_idx.shape[1]
    Hq, D = q.shape[2], q.shape[3]
    win, W = _window(win, (B, T), D)
    if lengths is not None:
        lengths = _c(lengths, np.int32)
        assert lengths.shape == (B, T)
    scores = np.empty((B, T, N), np.float32)
    idx = np.empty((B, T, k), np.int32)
    out = np.empty((B, T, Hq, D), np.float64)
    rc = _load().oracle_step_mt(_ptr(q_idx), _ptr(k_idx), _ptr(w), _ptr(q), _ptr(kv), _ptr(win),
                                None if lengths is None else _ptr(lengths), _ptr(scores),
                                _ptr(idx), _ptr(out), B, T, N, H, DI, int(k), W, Hq, D,
                                float(scale))
    if rc != 0:
        raise ValueError("oracle_step_mt: invalid arguments")
    return scores, idx, out


def qproj(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Indexer query projection. x uint16 (bf16) [B, d_in], w uint16 [O, d_in]
    -> float64 [B, O] = x @ w^T with exact products and double sums."""
    x = _c(x, np.uint16)
    w = _c(w, np.uint16)
    B, d_in = x.shape
    O = w.shape[0]
    assert w.shape == (O, d_in)
    out = np.empty((B, O), np.float64)
    _load().oracle_qproj(_ptr(x), _ptr(w), _ptr(out), B, d_in, O)
    return out


def compress(x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """Compressor: each group of 4 consecutive raw rows becomes one row,
    weighted by the softmax of the rows' gate scores wg . x_i. x uint16
    (bf16) [B, 4G, D], wg float32 [D] -> float64 [B, G, D]."""
    x = _c(x, np.uint16)
    wg = _c(wg, np.float32)
    B, R, D = x.shape
    if R % 4 != 0:
        raise ValueError("the raw rows must come in groups of 4")
    assert wg.shape == (D,)
    G = R // 4
    out = np.empty((B, G, D), np.float64)
    _load().oracle_compress(_ptr(x), _ptr(wg), _ptr(out), B, G, D)
    return out
