"""Build libidx.so for gfx950 in-tree: hipcc -shared over csrc/idx.hip."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "idx.hip")
OUT = os.path.join(HERE, "libidx.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    """Compile every time it is called; returns the library path."""
    tmp = OUT + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed for " + SRC)
    if verbose:
        sys.stderr.write(res.stderr)
    shutil.move(tmp, OUT)
    return OUT


def ensure_built() -> str:
    """Build only when no library exists yet (tests, smoke and bench call this)."""
    if not os.path.exists(OUT):
        build()
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
