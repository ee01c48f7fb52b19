"""Hardware probes used by the tests: built from source here, loaded with ctypes.

mfma_accum.hip measures how gfx950's matrix instructions accumulate (C = A·Bᵀ over
E4M3 or bf16 operands).  It is test infrastructure and not part of libidx."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mfma_accum.hip")
OUT = os.path.join(HERE, "libmfma_accum.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build() -> str:
    """Compile the probe library (every call)."""
    tmp = OUT + ".tmp"
    res = subprocess.run([HIPCC] + FLAGS + ["-o", tmp, SRC], capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed for " + SRC)
    shutil.move(tmp, OUT)
    return OUT


def load():
    """The probe library with its one entry point typed (built first if absent or older
    than its source)."""
    if not os.path.exists(OUT) or os.path.getmtime(OUT) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(OUT)
    f = lib.mfma_probe
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    return lib
