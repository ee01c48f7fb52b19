"""Synthetic index-cache workloads shaped like the GLM-5.3 indexer launch.

The GLM-5.3 indexer page (sgl-amd-mono-upstream pull request 18),
Modifications item 0 ("An exact top-k check"), checks the indexer on random keys, on four
keys repeated over every position (ties), on all-zero keys and on keys whose
last 4,096 positions are scaled 8x (recent), with served decode rows, mixed
rows and draft chains.  The configurations below take those shapes:

* queries bf16 drawn N(0, 1), head weights bf16 drawn N(0, 1/64) (sigma 1/8);
* keys f32 N(0, 1) per position, quantised per key to OCP FP8-E4M3FN with an
  f32 scale amax/448 (the usual per-token FP8 rule: divide by the scale,
  clamp to +-448, round to nearest even);
* pages of 64 keys; each request owns a seeded random permutation of pages.

Values are drawn with numpy's default_rng(seed) in the order q, w, keys (or
the four distinct key vectors), then the page permutation.  bf16 and FP8
rounding use torch's CPU casts; nothing here scores or selects.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

HEADS = 64
DIM = 128
PAGE = 64
TOPK = 2048
E4M3_MAX = 448.0


@dataclasses.dataclass
class Problem:
    """One call's worth of host-side inputs (all numpy, C-contiguous)."""

    name: str
    q: np.ndarray            # uint16 [rows, heads, dim]  (bf16 bit patterns)
    w: np.ndarray            # uint16 [rows, heads]       (bf16 bit patterns)
    k_cache: np.ndarray      # uint8  [num_pages, page_size, dim]  (E4M3FN codes)
    k_scale: np.ndarray      # float32 [num_pages, page_size]
    page_table: np.ndarray   # int32 [rows, max_pages]
    n_keys: np.ndarray       # int32 [rows]
    req_indptr: np.ndarray   # int32 [num_req + 1]
    k: int
    seed: int
    heads: int = HEADS
    dim: int = DIM
    page_size: int = PAGE

    @property
    def rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_req(self) -> int:
        return int(self.req_indptr.shape[0] - 1)

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def max_keys(self) -> int:
        return int(self.n_keys.max()) if self.rows else 0

    def key_rows(self) -> int:
        return int(self.n_keys.astype(np.int64).sum())


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round f32 to bf16 (nearest even) and return the 16-bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def quantize_keys(keys: np.ndarray):
    """Per-key FP8-E4M3FN quantisation: scale = f32(amax/448), codes of clamp(k/scale)."""
    keys = np.ascontiguousarray(keys, dtype=np.float32)
    amax = np.abs(keys).max(axis=-1)
    scale = amax / np.float32(E4M3_MAX)                      # f32 division
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32, copy=False)
    x = keys / safe[..., None]                               # f32, IEEE division
    np.clip(x, -E4M3_MAX, E4M3_MAX, out=x)
    x[scale == 0] = 0.0
    codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale.astype(np.float32, copy=False)


def make_problem(contexts: Sequence[int], rows_per_req: Sequence[int], *, seed: int,
                 k: int = TOPK, keys: str = "normal", recent: int = 4096,
                 recent_factor: float = 8.0, name: str = "custom",
                 heads: int = HEADS, dim: int = DIM, page: int = PAGE,
                 chain: bool = True, pad_pages: int = 0) -> Problem:
    """Build a problem with one request per entry of ``contexts``.

    Request j has ``rows_per_req[j]`` rows.  With ``chain`` its row i (of R)
    sees ``context - (R - 1) + i`` keys (an MTP verify chain over the shared
    pages); without it every row sees the whole context.  ``keys`` selects the
    cache: "normal", "ties" (four distinct vectors, position p carries vector
    p mod 4), "zeros", or "recent" (normal, with positions >= context - recent
    scaled by ``recent_factor`` before quantisation).  All requests' pages sit
    in one pool, permuted once and cut in request order.
    """
    rng = np.random.default_rng(seed)
    contexts = [int(c) for c in contexts]
    rows_per_req = [int(r) for r in rows_per_req]
    assert len(contexts) == len(rows_per_req)
    rows = sum(rows_per_req)
    q = bf16_bits(rng.standard_normal((rows, heads, dim), dtype=np.float32))
    w = bf16_bits((rng.standard_normal((rows, heads), dtype=np.float32) / np.float32(8.0)).astype(np.float32))

    req_pages = [(c + page - 1) // page for c in contexts]
    total_pages = max(1, sum(req_pages) + pad_pages)   # an empty pool still holds one page
    k_cache = np.zeros((total_pages, page, dim), dtype=np.uint8)
    k_scale = np.zeros((total_pages, page), dtype=np.float32)

    per_req_keys = []
    for c in contexts:
        if keys == "normal" or keys == "recent":
            kv = rng.standard_normal((c, dim), dtype=np.float32)
            if keys == "recent":
                lo = max(0, c - recent)
                kv[lo:] *= np.float32(recent_factor)
            codes, scale = quantize_keys(kv)
        elif keys == "ties":
            base = rng.standard_normal((4, dim), dtype=np.float32)
            bcodes, bscale = quantize_keys(base)
            idx = np.arange(c) % 4
            codes, scale = bcodes[idx], bscale[idx]
        elif keys == "zeros":
            codes = np.zeros((c, dim), dtype=np.uint8)
            scale = np.zeros((c,), dtype=np.float32)
        else:
            raise ValueError(keys)
        per_req_keys.append((codes, scale))

    perm_all = rng.permutation(total_pages).astype(np.int64)
    max_pages = max(req_pages) if req_pages else 0
    page_table = np.zeros((rows, max(1, max_pages)), dtype=np.int32)
    n_keys = np.zeros((rows,), dtype=np.int32)
    req_indptr = np.zeros((len(contexts) + 1,), dtype=np.int32)
    cut = 0
    r0 = 0
    for j, (c, R) in enumerate(zip(contexts, rows_per_req)):
        phys_pages = perm_all[cut: cut + req_pages[j]]
        cut += req_pages[j]
        codes, scale = per_req_keys[j]
        # logical page i of request j lives at physical page phys_pages[i]
        for i in range(req_pages[j]):
            lo, hi = i * page, min(c, (i + 1) * page)
            k_cache[phys_pages[i], : hi - lo] = codes[lo:hi]
            k_scale[phys_pages[i], : hi - lo] = scale[lo:hi]
        for i in range(R):
            page_table[r0 + i, : req_pages[j]] = phys_pages
            n_keys[r0 + i] = max(0, c - (R - 1) + i) if chain else c
        r0 += R
        req_indptr[j + 1] = r0
    return Problem(name=name, q=q, w=w, k_cache=k_cache, k_scale=k_scale,
                   page_table=page_table, n_keys=n_keys, req_indptr=req_indptr,
                   k=k, seed=seed, heads=heads, dim=dim, page_size=page)


CONFIG_NAMES = ["c0", "c1", "c2", "c3", "c4a", "c4b", "c4c"]

# Full-size recipes.  c0: one row over 4,096 keys.  c1: 4 verify rows over an
# 8,192-key context.  c2: 4 verify rows over 131,072 keys.  c3: 4 requests x 4
# rows with contexts 1,500 / 8,192 / 32,768 / 131,072.  c4a/b/c: the tie,
# zero and recent caches at 131,072 keys x 4 rows.
FULL_CONFIGS = {
    "c0": dict(contexts=[4096], rows_per_req=[1], seed=0),
    "c1": dict(contexts=[8192], rows_per_req=[4], seed=1),
    "c2": dict(contexts=[131072], rows_per_req=[4], seed=2),
    "c3": dict(contexts=[1500, 8192, 32768, 131072], rows_per_req=[4, 4, 4, 4], seed=3),
    "c4a": dict(contexts=[131072], rows_per_req=[4], seed=40, keys="ties"),
    "c4b": dict(contexts=[131072], rows_per_req=[4], seed=41, keys="zeros"),
    "c4c": dict(contexts=[131072], rows_per_req=[4], seed=42, keys="recent"),
}


def make_config(name: str, *, scale_down: Optional[int] = None) -> Problem:
    """The named configuration; ``scale_down`` divides every context (for CPU tests)."""
    spec = dict(FULL_CONFIGS[name])
    if scale_down:
        spec["contexts"] = [max(1, c // scale_down) for c in spec["contexts"]]
        if spec.get("keys") == "recent":
            spec["recent"] = max(1, 4096 // scale_down)
    return make_problem(name=name if not scale_down else f"{name}/{scale_down}", **spec)


def rope_table(positions, rope_dim: int, theta: float = 10000.0):
    """A RoPE rotation table for rows at the given positions: (cos, sin), f32
    [rows, rope_dim / 2], angle position * theta ** (-2 i / rope_dim) for pair i,
    evaluated in f64 and rounded to f32 (a caller-side input of query preparation)."""
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    i = np.arange(rope_dim // 2, dtype=np.float64)[None, :]
    ang = pos * theta ** (-2.0 * i / max(rope_dim, 1))
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
