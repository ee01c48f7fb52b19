"""ctypes declarations of libidx.so (include/idx.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libidx.so")

IDX_HEADS = 64
IDX_DIM = 128
IDX_PAGE_SIZE = 64
IDX_KMAX = 2048
IDX_GROUP_ROWS = 4
IDX_MAX_REQ = 256
IDX_MAX_KEYS = 1 << 28
IDX_NOALLOC_SCRATCH_BYTES = 16 << 20
IDX_ABI_VERSION = 3

IDX_OK = 0
IDX_EINVAL = 1
IDX_EUNSUPPORTED = 2
IDX_EWORKSPACE = 3
IDX_EHIP = 4
IDX_EDEVICE = 5
IDX_ESCRATCH = 6

IDX_DERR_NKEYS = 0x1
IDX_DERR_PAGE = 0x2
IDX_DERR_WS = 0x4
IDX_DERR_SELECT = 0x10

# every function the header declares, with its ctypes signature
_i32, _i64, _sz, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p


class IdxProblem(ctypes.Structure):
    _fields_ = [
        ("rows", _i32),
        ("num_req", _i32),
        ("req_indptr", ctypes.POINTER(_i32)),
        ("heads", _i32),
        ("dim", _i32),
        ("page_size", _i32),
        ("num_pages", _i32),
        ("max_pages", _i32),
        ("max_keys", _i32),
        ("q", _vp),
        ("w", _vp),
        ("k_cache", _vp),
        ("k_scale", _vp),
        ("page_table", _vp),
        ("n_keys", _vp),
        ("req_max_keys", ctypes.POINTER(_i32)),
    ]


class IdxNewKeys(ctypes.Structure):
    _fields_ = [("codes", _vp), ("scales", _vp), ("pos", _vp)]


SIGNATURES = {
    "idx_abi_version": (ctypes.c_int, []),
    "idx_workspace_bytes": (ctypes.c_int, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "idx_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "idx_score": (ctypes.c_int, [ctypes.POINTER(IdxProblem), _vp, _i64, _vp, _sz, _vp]),
    "idx_topk": (ctypes.c_int, [_vp, _i64, _vp, _i32, _i32, _i32, _vp, _vp, _sz, _vp]),
    "idx_score_topk": (ctypes.c_int, [ctypes.POINTER(IdxProblem), _i32, _vp, _i64, _vp, _vp, _sz, _vp]),
    "idx_score_topk_append": (ctypes.c_int, [ctypes.POINTER(IdxProblem), ctypes.POINTER(IdxNewKeys), _i32, _vp, _i64,
                                             _vp, _vp, _sz, _vp]),
    "idx_score_topk_slots": (ctypes.c_int, [ctypes.POINTER(IdxProblem), _i32, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "idx_score_topk_tagged": (ctypes.c_int, [ctypes.POINTER(IdxProblem), _i32, _vp, _i64, _vp, _vp, ctypes.c_uint32,
                                             _vp, _sz, _vp]),
    "idx_score_topk_noalloc": (ctypes.c_int, [ctypes.POINTER(IdxProblem), _i32, _vp, _i64, _vp, _vp]),
    "idx_prep_query": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp]),
    "idx_device_status": (ctypes.c_int, [_vp, _sz, _vp, ctypes.POINTER(ctypes.c_uint32)]),
    "idx_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "idx_last_hip_error": (ctypes.c_char_p, []),
    "idx_build_hash": (ctypes.c_char_p, []),
}

_lib = None


def load_file(path: str):
    """Load a build of the library from `path` with every signature declared (uncached)."""
    if not os.path.exists(path):
        raise ImportError(f"libidx.so is not built ({path}); run key_scoring_exact_amd.build.build()")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path: str = LIB_PATH):
    """Load libidx.so (built by key_scoring_exact_amd.build); raise if it is missing."""
    global _lib
    if _lib is None:
        _lib = load_file(path)
    return _lib
