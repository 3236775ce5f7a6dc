"""Builds libdsa.so (the HIP kernels and the C ABI of include/dsa.h) in-tree
for gfx950 with hipcc.

This module imports nothing from the package, so it can be run (or loaded by
path) before libdsa.so exists: `python indexer_top_gathered_amd/build.py`.
Each source is compiled to an object in a temporary folder, in parallel, and
the objects are linked into the shared library, which then replaces the old
one in one rename.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["topk.hip", "sparse_attend.hip", "indexer_score.hip", "dsa_api.hip", "qproj.hip",
           "compress.hip"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # Keep the compiler from forming packed-fp32 instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wno-unused-command-line-argument",
]


def _run(cmd):
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libdsa.so (always recompiles)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    jobs = jobs or max(1, min(len(SOURCES), len(os.sched_getaffinity(0))))
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmpdir:
        objs = [os.path.join(tmpdir, s + ".o") for s in SOURCES]
        cmds = [[hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for src, res in zip(SOURCES, results):
            if res.returncode != 0:
                sys.stderr.write(res.stdout + res.stderr)
                raise RuntimeError(f"hipcc failed on {src}")
            if verbose:
                sys.stderr.write(res.stderr)
        tmp = LIB + ".tmp%d" % os.getpid()
        res = _run([hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp])
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("linking libdsa.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
