"""MI355X sparse-attention indexer: exact key scoring and exact top-k (Python binding).

A thin ctypes layer over libidx.so (include/idx.h).  Every step runs in the HIP
kernels; this module only turns torch tensors into device pointers, picks the
current HIP stream and raises on error codes.  torch provides device memory and
streams.  There is no CPU fallback: without the built library, import of the
entry points fails loudly.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib
from ._lib import (IDX_DIM, IDX_GROUP_ROWS, IDX_HEADS, IDX_KMAX, IDX_MAX_REQ,  # noqa: F401
                   IDX_PAGE_SIZE, IdxProblem)

__all__ = ["IdxError", "DeviceProblem", "Workspace", "score", "topk", "score_topk", "score_topk_append",
           "score_topk_slots", "score_topk_tagged", "score_topk_noalloc", "prep_query", "device_status",
           "workspace_bytes", "lib"]


class IdxError(RuntimeError):
    def __init__(self, code: int, where: str):
        L = lib()
        msg = L.idx_strerror(code).decode()
        if code == _lib.IDX_EHIP:
            msg += ": " + L.idx_last_hip_error().decode()
        super().__init__(f"{where}: {msg} (code {code})")
        self.code = code


def lib():
    return _lib.load()


def _check(code: int, where: str):
    if code != _lib.IDX_OK:
        raise IdxError(code, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _shape(t: torch.Tensor, want, name: str):
    """Raise ValueError unless t has the given shape (None entries match any size)."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        raise ValueError(f"{name}: expected shape {tuple('*' if w is None else w for w in want)}, got {got}")


def _rows_at_least(t: torch.Tensor, rows: int, name: str):
    if t.dim() != 2 or t.shape[0] < rows:
        raise ValueError(f"{name}: expected a 2-D tensor of at least {rows} rows, got shape {tuple(t.shape)}")


def _ptr(t: torch.Tensor, dtype=None) -> int:
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"expected dtype {dtype}, got {t.dtype}")
    return t.data_ptr()


def workspace_bytes(rows: int, max_keys: int, k: int = IDX_KMAX) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().idx_workspace_bytes(int(rows), int(max_keys), int(k), ctypes.byref(out)), "idx_workspace_bytes")
    return int(out.value)


class Workspace:
    """Caller-owned device workspace (torch memory), initialised on creation."""

    def __init__(self, rows: int, max_keys: int, k: int = IDX_KMAX, device="cuda", stream=None):
        nbytes = workspace_bytes(rows, max_keys, k)
        self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        self.offset = (-base) % 256
        self.nbytes = nbytes
        self.reset(stream)

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + self.offset

    def reset(self, stream=None):
        _check(lib().idx_workspace_init(ctypes.c_void_p(self.ptr), self.nbytes, ctypes.c_void_p(_stream(stream))),
               "idx_workspace_init")


@dataclasses.dataclass
class DeviceProblem:
    """Device-resident inputs of one call; req_indptr (and req_max_keys) stay on the host."""

    q: torch.Tensor           # bf16 (or int16 bit patterns) [rows, 64, 128]
    w: torch.Tensor           # bf16 (or int16) [rows, 64]
    k_cache: torch.Tensor     # uint8 [num_pages, 64, 128] (E4M3FN codes)
    k_scale: torch.Tensor     # float32 [num_pages, 64]
    page_table: torch.Tensor  # int32 [rows, max_pages]
    n_keys: torch.Tensor      # int32 [rows]
    req_indptr: Sequence[int]
    max_keys: int
    req_max_keys: Optional[Sequence[int]] = None

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])

    @classmethod
    def from_arrays(cls, q, w, k_cache, k_scale, page_table, n_keys, req_indptr, max_keys=None,
                    req_max_keys=None, device="cuda") -> "DeviceProblem":
        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)

        n_keys = np.asarray(n_keys, dtype=np.int32)
        if max_keys is None:
            max_keys = int(n_keys.max()) if n_keys.size else 0
        return cls(q=up(q, np.int16), w=up(w, np.int16), k_cache=up(k_cache, np.uint8),
                   k_scale=up(k_scale, np.float32), page_table=up(page_table, np.int32),
                   n_keys=up(n_keys, np.int32), req_indptr=[int(x) for x in req_indptr],
                   max_keys=int(max_keys),
                   req_max_keys=None if req_max_keys is None else [int(x) for x in req_max_keys])

    def check_shapes(self):
        """Raise ValueError when the tensors' shapes disagree with each other: every
        kernel indexes them by rows, heads, dim and page size, so a short tensor would
        be read past its end."""
        if self.q.dim() != 3:
            raise ValueError(f"q: expected [rows, heads, dim], got shape {tuple(self.q.shape)}")
        rows, heads, dim = (int(x) for x in self.q.shape)
        _shape(self.w, (rows, heads), "w")
        if self.k_cache.dim() != 3 or int(self.k_cache.shape[2]) != dim:
            raise ValueError(f"k_cache: expected [num_pages, page_size, {dim}], got {tuple(self.k_cache.shape)}")
        _shape(self.k_scale, tuple(int(x) for x in self.k_cache.shape[:2]), "k_scale")
        _shape(self.page_table, (rows, None), "page_table")
        _shape(self.n_keys, (rows,), "n_keys")
        ip = list(self.req_indptr)
        if len(ip) < 2 or ip[0] != 0 or ip[-1] != rows or any(b <= a for a, b in zip(ip[:-1], ip[1:])):
            raise ValueError(f"req_indptr must rise strictly from 0 to rows={rows}, got {ip}")
        if self.req_max_keys is not None and len(self.req_max_keys) != len(ip) - 1:
            raise ValueError("req_max_keys: one bound a request expected")
        if self.max_keys > int(self.page_table.shape[1]) * int(self.k_cache.shape[1]):
            raise ValueError("max_keys exceeds the page table's capacity (max_pages * page_size)")

    def struct(self):
        """The idx_problem struct and the host arrays it points to (keep both alive)."""
        self.check_shapes()
        ip = (ctypes.c_int32 * len(self.req_indptr))(*self.req_indptr)
        rm = None
        if self.req_max_keys is not None:
            rm = (ctypes.c_int32 * len(self.req_max_keys))(*self.req_max_keys)
        s = IdxProblem(
            rows=self.rows, num_req=len(self.req_indptr) - 1,
            req_indptr=ctypes.cast(ip, ctypes.POINTER(ctypes.c_int32)),
            heads=int(self.q.shape[1]), dim=int(self.q.shape[2]), page_size=int(self.k_cache.shape[1]),
            num_pages=int(self.k_cache.shape[0]), max_pages=int(self.page_table.shape[1]),
            max_keys=int(self.max_keys),
            q=_ptr(self.q, (torch.bfloat16, torch.int16)), w=_ptr(self.w, (torch.bfloat16, torch.int16)),
            k_cache=_ptr(self.k_cache, (torch.uint8, torch.float8_e4m3fn)),
            k_scale=_ptr(self.k_scale, torch.float32),
            page_table=_ptr(self.page_table, torch.int32), n_keys=_ptr(self.n_keys, torch.int32),
            req_max_keys=None if rm is None else ctypes.cast(rm, ctypes.POINTER(ctypes.c_int32)))
        return s, (ip, rm)


def score(p: DeviceProblem, ws: Workspace, scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """f32 scores [rows, ld]; entries at positions >= n_keys[r] are left untouched."""
    if scores is None:
        scores = torch.empty((p.rows, max(1, p.max_keys)), dtype=torch.float32, device=p.q.device)
    _rows_at_least(scores, p.rows, "scores")
    s, keep = p.struct()
    _check(lib().idx_score(ctypes.byref(s), ctypes.c_void_p(_ptr(scores, torch.float32)), scores.shape[1],
                           ctypes.c_void_p(ws.ptr), ws.nbytes, ctypes.c_void_p(_stream(stream))), "idx_score")
    return scores


def score_topk(p: DeviceProblem, k: int, ws: Workspace, scores: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None, stream=None):
    """(scores [rows, ld] f32, lists [rows, k] int32) in one launch."""
    if scores is None:
        scores = torch.empty((p.rows, max(1, p.max_keys)), dtype=torch.float32, device=p.q.device)
    if out is None:
        out = torch.empty((p.rows, k), dtype=torch.int32, device=p.q.device)
    _rows_at_least(scores, p.rows, "scores")
    _shape(out, (p.rows, k), "out")
    s, keep = p.struct()
    _check(lib().idx_score_topk(ctypes.byref(s), int(k), ctypes.c_void_p(_ptr(scores, torch.float32)),
                                scores.shape[1], ctypes.c_void_p(_ptr(out, torch.int32)),
                                ctypes.c_void_p(ws.ptr), ws.nbytes, ctypes.c_void_p(_stream(stream))),
           "idx_score_topk")
    return scores, out


def score_topk_append(p: DeviceProblem, k: int, ws: Workspace, new_codes: torch.Tensor, new_scales: torch.Tensor,
                      new_pos: torch.Tensor, scores: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      stream=None):
    """(scores, lists) with every row's new key written in the same launch: new_codes uint8
    [rows, 128], new_scales f32 [rows], new_pos int32 [rows] (-1: none).  Writes the keys
    into p.k_cache / p.k_scale."""
    if scores is None:
        scores = torch.empty((p.rows, max(1, p.max_keys)), dtype=torch.float32, device=p.q.device)
    if out is None:
        out = torch.empty((p.rows, k), dtype=torch.int32, device=p.q.device)
    _rows_at_least(scores, p.rows, "scores")
    _shape(out, (p.rows, k), "out")
    _shape(new_codes, (p.rows, int(p.q.shape[2])), "new_codes")
    _shape(new_scales, (p.rows,), "new_scales")
    _shape(new_pos, (p.rows,), "new_pos")
    s, keep = p.struct()
    nk = _lib.IdxNewKeys(_ptr(new_codes, torch.uint8), _ptr(new_scales, torch.float32), _ptr(new_pos, torch.int32))
    _check(lib().idx_score_topk_append(ctypes.byref(s), ctypes.byref(nk), int(k),
                                       ctypes.c_void_p(_ptr(scores, torch.float32)), scores.shape[1],
                                       ctypes.c_void_p(_ptr(out, torch.int32)), ctypes.c_void_p(ws.ptr), ws.nbytes,
                                       ctypes.c_void_p(_stream(stream))), "idx_score_topk_append")
    return scores, out


def score_topk_slots(p: DeviceProblem, k: int, ws: Workspace, scores: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, slots: Optional[torch.Tensor] = None, stream=None):
    """(scores, lists, slots): as score_topk, plus each list as physical cache slots [rows, k]."""
    if scores is None:
        scores = torch.empty((p.rows, max(1, p.max_keys)), dtype=torch.float32, device=p.q.device)
    if out is None:
        out = torch.empty((p.rows, k), dtype=torch.int32, device=p.q.device)
    if slots is None:
        slots = torch.empty((p.rows, k), dtype=torch.int32, device=p.q.device)
    _rows_at_least(scores, p.rows, "scores")
    _shape(out, (p.rows, k), "out")
    _shape(slots, (p.rows, k), "slots")
    s, keep = p.struct()
    _check(lib().idx_score_topk_slots(ctypes.byref(s), int(k), ctypes.c_void_p(_ptr(scores, torch.float32)),
                                      scores.shape[1], ctypes.c_void_p(_ptr(out, torch.int32)),
                                      ctypes.c_void_p(_ptr(slots, torch.int32)), ctypes.c_void_p(ws.ptr), ws.nbytes,
                                      ctypes.c_void_p(_stream(stream))), "idx_score_topk_slots")
    return scores, out, slots


def score_topk_tagged(p: DeviceProblem, k: int, ws: Workspace, tag: int, scores: Optional[torch.Tensor] = None,
                      out: Optional[torch.Tensor] = None, tagged: Optional[torch.Tensor] = None, stream=None):
    """(scores, lists, tagged): as score_topk, plus each list's cache slots as 64-bit words
    tag << 32 | slot (int64 [rows, k]; slot -1 is stored as 0xFFFFFFFF)."""
    if scores is None:
        scores = torch.empty((p.rows, max(1, p.max_keys)), dtype=torch.float32, device=p.q.device)
    if out is None:
        out = torch.empty((p.rows, k), dtype=torch.int32, device=p.q.device)
    if tagged is None:
        tagged = torch.empty((p.rows, k), dtype=torch.int64, device=p.q.device)
    _rows_at_least(scores, p.rows, "scores")
    _shape(out, (p.rows, k), "out")
    _shape(tagged, (p.rows, k), "tagged")
    if not 0 <= int(tag) < (1 << 32):
        raise ValueError("tag must fit 32 bits")
    s, keep = p.struct()
    _check(lib().idx_score_topk_tagged(ctypes.byref(s), int(k), ctypes.c_void_p(_ptr(scores, torch.float32)),
                                       scores.shape[1], ctypes.c_void_p(_ptr(out, torch.int32)),
                                       ctypes.c_void_p(_ptr(tagged, torch.int64)), int(tag), ctypes.c_void_p(ws.ptr),
                                       ws.nbytes, ctypes.c_void_p(_stream(stream))), "idx_score_topk_tagged")
    return scores, out, tagged


def score_topk_noalloc(p: DeviceProblem, k: int, scores: torch.Tensor, out: torch.Tensor, stream=None):
    """idx_score_topk_noalloc: as score_topk, with the library's static per-device scratch in
    place of a workspace; the caller passes the output tensors (nothing is allocated)."""
    _rows_at_least(scores, p.rows, "scores")
    _shape(out, (p.rows, k), "out")
    s, keep = p.struct()
    _check(lib().idx_score_topk_noalloc(ctypes.byref(s), int(k), ctypes.c_void_p(_ptr(scores, torch.float32)),
                                        scores.shape[1], ctypes.c_void_p(_ptr(out, torch.int32)),
                                        ctypes.c_void_p(_stream(stream))), "idx_score_topk_noalloc")
    return scores, out


def topk(scores: torch.Tensor, n_keys: torch.Tensor, k: int, max_keys: int, ws: Workspace,
         out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Exact top-k lists [rows, k] int32 of given f32 scores [rows, ld]."""
    if scores.dim() != 2:
        raise ValueError(f"scores: expected [rows, ld], got shape {tuple(scores.shape)}")
    rows = int(scores.shape[0])
    _shape(n_keys, (rows,), "n_keys")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    _shape(out, (rows, k), "out")
    _check(lib().idx_topk(ctypes.c_void_p(_ptr(scores, torch.float32)), scores.shape[1],
                          ctypes.c_void_p(_ptr(n_keys, torch.int32)), rows, int(max_keys), int(k),
                          ctypes.c_void_p(_ptr(out, torch.int32)), ctypes.c_void_p(ws.ptr), ws.nbytes,
                          ctypes.c_void_p(_stream(stream))), "idx_topk")
    return out


def prep_query(q_pre: torch.Tensor, cos: Optional[torch.Tensor], sin: Optional[torch.Tensor], rope_dim: int,
               interleaved: bool = False, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The prepared index query, bf16 [rows, 64, 128]: RoPE on the first rope_dim dims of
    every head from the per-row table cos / sin f32 [rows, rope_dim / 2] (half-split or
    interleaved pairs), then the orthonormal Hadamard transform; f32 arithmetic, bf16 out."""
    rows = int(q_pre.shape[0])
    if out is None:
        out = torch.empty_like(q_pre)
    if q_pre.dim() != 3 or tuple(q_pre.shape[1:]) != (IDX_HEADS, IDX_DIM) or out.shape != q_pre.shape:
        raise ValueError("expected q_pre and out of shape [rows, 64, 128]")
    if rope_dim > 0:
        _shape(cos, (rows, int(rope_dim) // 2), "cos")
        _shape(sin, (rows, int(rope_dim) // 2), "sin")
    cp = ctypes.c_void_p(_ptr(cos, torch.float32)) if rope_dim > 0 else None
    sp = ctypes.c_void_p(_ptr(sin, torch.float32)) if rope_dim > 0 else None
    bf = (torch.bfloat16, torch.int16)
    _check(lib().idx_prep_query(ctypes.c_void_p(_ptr(q_pre, bf)), cp, sp, rows, int(rope_dim),
                                1 if interleaved else 0, ctypes.c_void_p(_ptr(out, bf)),
                                ctypes.c_void_p(_stream(stream))), "idx_prep_query")
    return out


def device_status(ws: Workspace, stream=None):
    """(code, detail bits): synchronises the stream, reads and clears the sticky error."""
    detail = ctypes.c_uint32(0)
    code = lib().idx_device_status(ctypes.c_void_p(ws.ptr), ws.nbytes, ctypes.c_void_p(_stream(stream)),
                                   ctypes.byref(detail))
    return int(code), int(detail.value)

