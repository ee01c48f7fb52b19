"""Hardware probes used by the tests: built from source here, loaded with ctypes.

mfma_accum.hip measures how gfx950's matrix instructions accumulate (C = A·Bᵀ over E4M3
or bf16 operands); xcd_coherence.hip measures which cache-policy bits make one
workgroup's stores visible to a workgroup on another XCD within the same launch.  They
are test infrastructure and not part of libidx."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
PROBES = {"mfma_accum": ("mfma_probe", [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
          "mfma_rate": ("mfma_rate", [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_double)]),
          "xcd_coherence": ("xcd_coherence_probe", [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                    ctypes.POINTER(ctypes.c_uint32),
                                                    ctypes.POINTER(ctypes.c_uint32)])}


LIBS = {"mfma_rate": "mfma_accum"}          # entry points that live in another probe's library


def _paths(name):
    name = LIBS.get(name, name)
    return os.path.join(HERE, name + ".hip"), os.path.join(HERE, "lib" + name + ".so")


def build(names=("mfma_accum", "xcd_coherence")) -> None:
    """Compile the probe libraries (every call)."""
    for name in names:
        src, out = _paths(name)
        tmp = out + ".tmp"
        res = subprocess.run([HIPCC] + FLAGS + ["-o", tmp, src], capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed for " + src)
        shutil.move(tmp, out)


def load(name="mfma_accum"):
    """A probe library with its entry point typed (built first if absent or older than
    its source)."""
    src, out = _paths(name)
    if not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        build([name])
    lib = ctypes.CDLL(out)
    fname, argtypes = PROBES[name]
    f = getattr(lib, fname)
    f.argtypes = argtypes
    f.restype = ctypes.c_int
    return lib
