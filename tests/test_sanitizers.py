"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code.

The CPU oracle (oracle.c) is built with gcc and the sanitizers together with
tests/sanitize/oracle_driver.c, which calls every oracle function on small
inputs. The library's host code (argument checks, plans and workspace
layouts in the HIP sources) is built with hipcc, the sanitizers given to the
host pass only (-Xarch_host; the GPU code is built as usual and never runs
here), together with tests/sanitize/abi_driver.cpp, which calls every entry
point over a grid of valid and invalid shapes with fake pointers. Both must
run clean: any sanitizer report aborts the program with a non-zero status.
CPU only."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "indexer_top_gathered_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
                    "-o", exe, "-lm"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "0 failed checks" in res.stdout


def test_library_host_code_under_asan_ubsan(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("the driver's valid shapes would launch kernels on fake pointers")
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    flags = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Wno-unused-command-line-argument"]
    srcs = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")]
    srcs.append(os.path.join(HERE, "abi_driver.cpp"))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        r = subprocess.run([hipcc, *flags, *lang, "-c", src, "-o", obj], capture_output=True,
                           text=True)
        return obj, r

    with ThreadPoolExecutor(min(len(srcs), max(1, len(os.sched_getaffinity(0))))) as ex:
        built = list(ex.map(compile_one, srcs))
    for (obj, r), src in zip(built, srcs):
        assert r.returncode == 0, f"{src}: {r.stderr[-3000:]}"
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", *[o for o, _ in built], "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "0 unexpected statuses" in res.stdout
