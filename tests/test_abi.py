"""C-ABI checks that need no GPU: the library loads, exports every entry
point include/dsa.h declares, and rejects bad arguments on the host before
touching a device."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIB_PATH = os.path.join(ROOT, "indexer_top_gathered_amd", "libdsa.so")

SUCCESS, INVALID, NOT_SUPPORTED, WS_SMALL, LAUNCH, DEVICE, SCRATCH_LIMIT = range(7)


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DSA_EXPORT[^;(]*?\b(dsa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_dsa_build", os.path.join(ROOT, "indexer_top_gathered_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    from indexer_top_gathered_amd import binding
    return binding


def test_header_declares_the_four_calls():
    syms = declared_symbols()
    for name in ("dsa_indexer_score", "dsa_topk", "dsa_sparse_attend", "dsa_decode_step"):
        assert name in syms


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(LIB_PATH)
    for name in declared_symbols():
        assert hasattr(raw, name), name
    assert set(declared_symbols()) == set(lib.EXPORTED)


def test_status_strings(lib):
    for s in range(7):
        assert lib.status_string(s).startswith("DSA_")
    assert "UNKNOWN" in lib.status_string(99)


P = 0x10000  # a fake, 16-byte aligned address: never dereferenced by these calls


def _dims(lib, **kw):
    base = dict(B=2, N=4096, H_I=8, D_I=128, k=256, W=64, H_q=16, D=128, scale=0.088)
    base.update(kw)
    return lib.make_dims(**base)


def test_indexer_argument_errors(lib):
    L = lib.LIB
    v = ctypes.c_void_p
    assert L.dsa_indexer_score(None, v(P), v(P), v(P), 1, 10, 8, 128, None) == INVALID
    assert L.dsa_indexer_score(v(P), v(P), v(P), v(P + 8), 1, 10, 8, 128, None) == INVALID
    assert L.dsa_indexer_score(v(P), v(P), v(P), v(P), 0, 10, 8, 128, None) == INVALID
    assert L.dsa_indexer_score(v(P), v(P), v(P), v(P), 1, 10, 8, 64, None) == NOT_SUPPORTED
    assert L.dsa_indexer_score(v(P), v(P), v(P), v(P), 1, 10, 65, 128, None) == NOT_SUPPORTED


def test_topk_argument_errors(lib):
    L = lib.LIB
    v = ctypes.c_void_p
    assert L.dsa_topk_workspace_bytes(4, 100, 101, 0) == 0
    assert L.dsa_topk_workspace_bytes(4, 100, 0, 1) == 0
    assert L.dsa_topk_workspace_bytes(4, 10000, 5000, 1) == 0  # k above 4096
    need = L.dsa_topk_workspace_bytes(4, 100000, 512, 0)
    assert need > 0
    assert L.dsa_topk(v(P), 0, 4, 100, 101, v(P), None, 0, v(P), 1 << 20, None) == INVALID
    assert L.dsa_topk(v(P), 2, 4, 100, 10, v(P), None, 0, v(P), 1 << 20, None) == INVALID
    assert L.dsa_topk(None, 0, 4, 100, 10, v(P), None, 0, v(P), 1 << 20, None) == INVALID
    assert L.dsa_topk(v(P + 2), 0, 4, 100, 10, v(P), None, 0, v(P), 1 << 20, None) == INVALID
    assert L.dsa_topk(v(P), 0, 4, 100, 10, v(P), None, 2, v(P), 1 << 20, None) == INVALID
    assert L.dsa_topk(v(P), 1, 4, 100, 10, v(P), v(P + 2), 0, v(P), 1 << 20, None) == INVALID
    assert L.dsa_topk(v(P), 0, 4, 100000, 512, v(P), None, 0, v(P), need - 1, None) == WS_SMALL
    assert L.dsa_topk(v(P), 0, 4, 10000, 5000, v(P), None, 0, v(P), 1 << 30, None) == NOT_SUPPORTED


def test_attend_and_step_argument_errors(lib):
    L = lib.LIB
    v = ctypes.c_void_p
    ok = _dims(lib)
    assert lib.dsa_sparse_attend_workspace_bytes(ok) > 0
    assert lib.dsa_decode_step_workspace_bytes(ok) > 0
    for bad, code in [(dict(D=64), NOT_SUPPORTED), (dict(H_q=24), NOT_SUPPORTED),
                      (dict(H_q=144), NOT_SUPPORTED), (dict(k=5000, N=6000), NOT_SUPPORTED),
                      (dict(k=0), INVALID), (dict(k=5000), INVALID), (dict(W=-1), INVALID),
                      (dict(scale=float("nan")), INVALID), (dict(B=0), INVALID)]:
        d = _dims(lib, **bad)
        assert lib.dsa_sparse_attend_workspace_bytes(d) == 0, bad
        assert L.dsa_sparse_attend(v(P), v(P), v(P), v(P), v(P), ctypes.byref(d), v(P), 1 << 30,
                                   None) == code, bad
    d = _dims(lib, D_I=64)
    assert lib.dsa_decode_step_workspace_bytes(d) == 0
    assert L.dsa_decode_step(v(P), v(P), v(P), v(P), v(P), v(P), v(P), None, ctypes.byref(d),
                             v(P), 1 << 30, None) == NOT_SUPPORTED
    # window rows promised but no window tensor
    assert L.dsa_sparse_attend(v(P), v(P), v(P), None, v(P), ctypes.byref(ok), v(P), 1 << 30,
                               None) == INVALID
    need = lib.dsa_decode_step_workspace_bytes(ok)
    assert L.dsa_decode_step(v(P), v(P), v(P), v(P), v(P), v(P), v(P), None, ctypes.byref(ok),
                             v(P), need - 1, None) == WS_SMALL
    assert L.dsa_decode_step(v(P), v(P), v(P), v(P), v(P), v(P), v(P + 4), None,
                             ctypes.byref(ok), v(P), need, None) == INVALID


def test_noalloc_argument_errors(lib):
    L = lib.LIB
    v = ctypes.c_void_p
    ok = _dims(lib)
    args = [v(P)] * 7 + [None]
    d = _dims(lib, D=64)
    assert L.dsa_decode_step_noalloc(*args, ctypes.byref(d), None) == NOT_SUPPORTED
    d = _dims(lib, k=0)
    assert L.dsa_decode_step_noalloc(*args, ctypes.byref(d), None) == INVALID
    assert L.dsa_decode_step_noalloc(*args, None, None) == INVALID
    bad = [v(P)] * 6 + [None, None]  # no output
    assert L.dsa_decode_step_noalloc(*bad, ctypes.byref(ok), None) == INVALID
    # the stress shape (64 x 262144) needs far more than the static scratch
    big = _dims(lib, B=64, N=262144, H_I=64, k=2048, W=128, H_q=128, D=512)
    assert lib.dsa_decode_step_workspace_bytes(big) > lib.NOALLOC_SCRATCH_BYTES
    assert L.dsa_decode_step_noalloc(*args, ctypes.byref(big), None) == SCRATCH_LIMIT
    # the production shape fits
    prod = _dims(lib, B=16, N=32768, H_I=64, k=1024, W=128, H_q=128, D=512)
    assert lib.dsa_decode_step_workspace_bytes(prod) <= lib.NOALLOC_SCRATCH_BYTES
    assert "DSA_NOALLOC_SCRATCH_BYTES (64u << 20)" in open(HEADER).read()


def test_sink_and_compress_argument_errors(lib):
    L = lib.LIB
    v = ctypes.c_void_p
    ok = _dims(lib)
    # no sink, or a misaligned one
    assert L.dsa_sparse_attend_sink(v(P), v(P), v(P), v(P), None, v(P), ctypes.byref(ok), v(P),
                                    1 << 30, None) == INVALID
    assert L.dsa_sparse_attend_sink(v(P), v(P), v(P), v(P), v(P + 2), v(P), ctypes.byref(ok),
                                    v(P), 1 << 30, None) == INVALID
    assert L.dsa_decode_step_sink(v(P), v(P), v(P), v(P), v(P), v(P), None, v(P), None,
                                  ctypes.byref(ok), v(P), 1 << 30, None) == INVALID
    need = lib.dsa_decode_step_workspace_bytes(ok)
    assert L.dsa_decode_step_sink(v(P), v(P), v(P), v(P), v(P), v(P), v(P), v(P), None,
                                  ctypes.byref(ok), v(P), need - 1, None) == WS_SMALL
    bad = _dims(lib, D=64)
    assert L.dsa_sparse_attend_sink(v(P), v(P), v(P), v(P), v(P), v(P), ctypes.byref(bad), v(P),
                                    1 << 30, None) == NOT_SUPPORTED
    # compressor
    assert L.dsa_compress(None, v(P), v(P), 1, 1, 512, None) == INVALID
    assert L.dsa_compress(v(P), v(P), v(P + 8), 1, 1, 512, None) == INVALID
    assert L.dsa_compress(v(P), v(P), v(P), 0, 1, 512, None) == INVALID
    assert L.dsa_compress(v(P), v(P), v(P), 1, 0, 512, None) == INVALID
    assert L.dsa_compress(v(P), v(P), v(P), 1, 1, 100, None) == NOT_SUPPORTED
    assert L.dsa_compress(v(P), v(P), v(P), 1, 1, 2048, None) == NOT_SUPPORTED


def test_indexer_topk_argument_errors(lib):
    L = lib.LIB
    v = ctypes.c_void_p
    need = L.dsa_indexer_topk_workspace_bytes(16, 32768, 64, 1024, 1)
    assert need > 0 and L.dsa_indexer_topk_workspace_bytes(16, 32768, 64, 1024, 0) < need
    assert L.dsa_indexer_topk_workspace_bytes(16, 32768, 64, 0, 1) == 0       # k < 1
    assert L.dsa_indexer_topk_workspace_bytes(16, 32768, 65, 1024, 1) == 0    # H_I > 64
    assert L.dsa_indexer_topk_chunks(16, 32768, 1024) == 16
    assert L.dsa_indexer_topk_chunks(16, 32768, 0) == 0
    # Rows that one top-k workgroup takes whole (N <= 8192) skip the cut.
    assert L.dsa_indexer_topk_chunks(1, 4096, 256) == 0
    assert L.dsa_indexer_topk_chunks(1, 8192, 256) == 0
    assert L.dsa_indexer_topk_chunks(1, 8193, 256) > 1
    args = (v(P), v(P), v(P), 16, 32768, 64, 128, 1024)
    assert L.dsa_indexer_topk(*args, None, None, v(P), need, None) == INVALID          # no out
    assert L.dsa_indexer_topk(*args, v(P + 2), None, v(P), need, None) == INVALID      # misaligned
    assert L.dsa_indexer_topk(*args, v(P), v(P + 4), v(P), need, None) == INVALID      # scores
    assert L.dsa_indexer_topk(*args, v(P), None, v(P), need - 1, None) == WS_SMALL
    assert L.dsa_indexer_topk(v(P), v(P), v(P), 16, 32768, 64, 64, 1024, v(P), None, v(P), need,
                              None) == NOT_SUPPORTED                                   # D_I != 128
    assert L.dsa_indexer_topk(v(P), v(P), v(P), 16, 1000, 64, 128, 1001, v(P), None, v(P), need,
                              None) == INVALID                                         # k > N


def test_valid_call_without_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is visible: this check is for hosts without one")
    L = lib.LIB
    v = ctypes.c_void_p
    assert L.dsa_indexer_score(v(P), v(P), v(P), v(P), 1, 10, 8, 128, None) == DEVICE
    assert L.dsa_decode_step_noalloc(*([v(P)] * 7), None, ctypes.byref(_dims(lib)),
                                     None) == DEVICE
    assert L.dsa_compress(v(P), v(P), v(P), 2, 3, 512, None) == DEVICE
    need = L.dsa_indexer_topk_workspace_bytes(2, 1000, 8, 64, 1)
    assert L.dsa_indexer_topk(v(P), v(P), v(P), 2, 1000, 8, 128, 64, v(P), None, v(P), need,
                              None) == DEVICE


def test_ragged_and_multi_token_argument_errors(lib):
    L = lib.LIB
    v = ctypes.c_void_p
    ok = _dims(lib)
    # ragged: lengths are required and 4-byte aligned
    assert L.dsa_topk_ragged(v(P), 0, 4, 100, None, 10, v(P), None, 0, v(P), 1 << 20,
                             None) == INVALID
    assert L.dsa_topk_ragged(v(P), 0, 4, 100, v(P + 2), 10, v(P), None, 0, v(P), 1 << 20,
                             None) == INVALID
    assert L.dsa_decode_step_ragged(v(P), v(P), v(P), v(P), v(P), v(P), None, v(P), None,
                                    ctypes.byref(ok), v(P), 1 << 30, None) == INVALID
    # several tokens: 1 <= T <= 4, B*T within the attention limit
    one = lib.dsa_decode_step_workspace_bytes(ok)
    assert L.dsa_decode_step_mt_workspace_bytes(ctypes.byref(ok), 1) == one
    assert L.dsa_sparse_attend_mt_workspace_bytes(ctypes.byref(ok), 1) == \
        lib.dsa_sparse_attend_workspace_bytes(ok)
    two = L.dsa_decode_step_mt_workspace_bytes(ctypes.byref(ok), 2)
    assert two > one
    for T in (0, 5):
        assert L.dsa_decode_step_mt_workspace_bytes(ctypes.byref(ok), T) == 0
        assert L.dsa_sparse_attend_mt_workspace_bytes(ctypes.byref(ok), T) == 0
    assert L.dsa_indexer_score_mt(v(P), v(P), v(P), v(P), 1, 0, 10, 8, 128, None) == INVALID
    assert L.dsa_indexer_score_mt(v(P), v(P), v(P), v(P), 1, 5, 10, 8, 128, None) == NOT_SUPPORTED
    assert L.dsa_indexer_score_mt(v(P), v(P), v(P), v(P + 8), 1, 2, 10, 8, 128, None) == INVALID
    assert L.dsa_sparse_attend_mt(v(P), v(P), v(P), v(P), v(P), ctypes.byref(ok), 5, v(P),
                                  1 << 30, None) == NOT_SUPPORTED
    assert L.dsa_decode_step_mt(v(P), v(P), v(P), v(P), v(P), v(P), None, v(P), None,
                                ctypes.byref(ok), 0, v(P), 1 << 30, None) == INVALID
    assert L.dsa_decode_step_mt(v(P), v(P), v(P), v(P), v(P), v(P), v(P + 2), v(P), None,
                                ctypes.byref(ok), 2, v(P), 1 << 30, None) == INVALID
    assert L.dsa_decode_step_mt(v(P), v(P), v(P), v(P), v(P), v(P), None, v(P), None,
                                ctypes.byref(ok), 2, v(P), two - 1, None) == WS_SMALL
    big = _dims(lib, B=20000)
    assert L.dsa_decode_step_mt_workspace_bytes(ctypes.byref(big), 4) == 0  # B*T > 65535


def test_package_import_fails_loudly_without_the_library(tmp_path):
    # A copy of the Python package with no libdsa.so beside it: importing it
    # must raise, never fall back to another implementation.
    import shutil
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "indexer_top_gathered_amd")
    dst = tmp_path / "indexer_top_gathered_amd"
    dst.mkdir()
    for name in ("__init__.py", "binding.py"):
        shutil.copy(os.path.join(pkg, name), dst / name)
    code = ("import sys; sys.path.insert(0, sys.argv[1])\n"
            "try:\n"
            "    import indexer_top_gathered_amd\n"
            "except ImportError as e:\n"
            "    print('ImportError:', e); sys.exit(3)\n"
            "sys.exit(0)\n")
    res = subprocess.run([sys.executable, "-c", code, str(tmp_path)], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 3, res.stdout + res.stderr
    assert "libdsa.so is missing" in res.stdout
