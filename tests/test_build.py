"""The build entry point works from a clean checkout: the tracked files alone,
with no libdsa.so and no liboracle.so, are copied to a temporary folder, and
`__graft_entry__.build()` there must compile both libraries and import the
package (whose import loads libdsa.so and fails when it is missing)."""
from __future__ import annotations

import ctypes
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILT = (".so", ".o", ".pyc")


def tracked_files():
    try:
        out = subprocess.run(["git", "-C", ROOT, "ls-files", "-z"], capture_output=True,
                             check=True).stdout
        files = [f for f in out.decode().split("\0") if f]
    except (OSError, subprocess.CalledProcessError):
        files = []
        for d, dirs, names in os.walk(ROOT):
            dirs[:] = [x for x in dirs if not x.startswith((".", "_work", "gpurun_out", "__pycache__"))]
            files += [os.path.relpath(os.path.join(d, n), ROOT) for n in names]
    return [f for f in files if not f.endswith(BUILT) and os.path.isfile(os.path.join(ROOT, f))]


def test_build_from_clean_checkout(tmp_path):
    for rel in tracked_files():
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy2(os.path.join(ROOT, rel), dst)
    assert not (tmp_path / "indexer_top_gathered_amd" / "libdsa.so").exists()
    res = subprocess.run([sys.executable, "-c", "import __graft_entry__ as e; e.build()"],
                         cwd=tmp_path, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    lib = tmp_path / "indexer_top_gathered_amd" / "libdsa.so"
    assert lib.exists() and (tmp_path / "oracle" / "liboracle.so").exists()
    header = (tmp_path / "include" / "dsa.h").read_text()
    raw = ctypes.CDLL(str(lib))
    for name in set(re.findall(r"DSA_EXPORT[^;(]*?\b(dsa_\w+)\s*\(", header)):
        assert hasattr(raw, name), name
