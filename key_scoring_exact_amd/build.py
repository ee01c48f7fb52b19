"""Build libidx.so for gfx950 in-tree: hipcc -shared over csrc/idx.hip.

The library carries the SHA-256 of what it was built from (csrc/idx.hip, include/idx.h
and the compiler flags), both as the return value of idx_build_hash() and as a marker
string in the file, so that a stale library is found without loading it."""
from __future__ import annotations

import hashlib
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "idx.hip")
HDR = os.path.join(ROOT, "include", "idx.h")
OUT = os.path.join(HERE, "libidx.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
MARKER = b"idx-source-sha256:"


def source_hash(extra_flags=()) -> str:
    """SHA-256 (hex) of the kernel source, the header and the compiler flags."""
    h = hashlib.sha256()
    for path in (SRC, HDR):
        h.update(open(path, "rb").read())
    h.update(" ".join(FLAGS[:-1] + list(extra_flags)).encode())
    return h.hexdigest()


def library_hash(path: str = OUT):
    """The source hash a built library carries, read from its bytes (None if absent)."""
    try:
        data = open(path, "rb").read()
    except OSError:
        return None
    m = re.search(re.escape(MARKER) + rb"([0-9a-f]{64})", data)
    return m.group(1).decode() if m else None


def build(verbose: bool = False, out: str = OUT, extra_flags=()) -> str:
    """Compile every time it is called; returns the library path."""
    tmp = out + ".tmp"
    digest = source_hash(extra_flags)
    cmd = [HIPCC] + FLAGS + list(extra_flags) + [f'-DIDX_SOURCE_HASH="{digest}"', "-o", tmp, SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed for " + SRC)
    if verbose:
        sys.stderr.write(res.stderr)
    shutil.move(tmp, out)
    return out


def ensure_built() -> str:
    """Build when no library exists or the one present was built from other sources
    (tests, smoke and bench call this before loading it)."""
    if library_hash(OUT) != source_hash():
        build()
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
