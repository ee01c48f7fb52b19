"""Checks of a GPU result against the CPU oracle.

TEST INFRASTRUCTURE ONLY (see oracle/indexer.py).

The checks restate those of the GLM-5.3 indexer page (sgl-amd-mono-upstream pull
request 18), Modifications item 0, in this project's terms:

* scores: compared with the f64 oracle; the largest absolute difference over a row,
  divided by the row's largest oracle score, may not exceed 1e-4.  "Largest" is read
  as the largest in magnitude, M_r = max_p |v[p]|; a row with M_r = 0 must match
  exactly;
* the list: compared entry by entry with the exact selection computed from the GPU's
  own scores, so a key that rounding puts on either side of the threshold cannot fail
  a correct kernel;
* "missed": the number of positions of the exact top-k of the oracle's scores that
  the GPU list does not contain (reported only);
* negative controls: three deliberately damaged copies of a row's result (one chosen
  position traded for the best position left out, two list entries exchanged, one
  bit of one score inverted), each of which the checks above must reject;
* SHA-256 digests of each row's scores and list, for comparing runs.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List

import numpy as np

from .indexer import select

SCORE_BOUND = 1e-4


@dataclasses.dataclass
class RowReport:
    row: int
    n: int
    err_over_max: float      # max |gpu - ref| / M_r (0 when M_r == 0 and exact)
    score_ok: bool
    list_ok: bool
    missed: int
    scores_digest: str
    list_digest: str


def score_error(gpu: np.ndarray, ref: np.ndarray):
    """(max |gpu-ref| / M, ok) over positions 0..n-1, M = max |ref|."""
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError("shape mismatch")
    if g.size == 0:
        return 0.0, True
    if not np.isfinite(g).all():
        return float("inf"), False
    m = float(np.max(np.abs(r)))
    d = float(np.max(np.abs(g - r)))
    if m == 0.0:
        return (0.0 if d == 0.0 else float("inf")), d == 0.0
    return d / m, d <= SCORE_BOUND * m


def list_exact(gpu_list: np.ndarray, gpu_scores: np.ndarray, n: int, k: int) -> bool:
    """The list equals the exact selection over the GPU's own scores, entry by entry."""
    want = select(np.asarray(gpu_scores, dtype=np.float64), n, k)
    return bool(np.array_equal(np.asarray(gpu_list, dtype=np.int32), want))


def missed(gpu_list: np.ndarray, ref_scores: np.ndarray, n: int, k: int) -> int:
    want = select(ref_scores, n, k)
    want = set(int(x) for x in want if x >= 0)
    have = set(int(x) for x in gpu_list if x >= 0)
    return len(want - have)


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def check_row(r: int, gpu_scores: np.ndarray, gpu_list: np.ndarray,
              ref_scores: np.ndarray, n: int, k: int) -> RowReport:
    e, ok = score_error(gpu_scores[:n], ref_scores[:n])
    return RowReport(row=r, n=n, err_over_max=e, score_ok=ok,
                     list_ok=list_exact(gpu_list, gpu_scores[:n], n, k),
                     missed=missed(gpu_list, ref_scores[:n], n, k),
                     scores_digest=digest(np.asarray(gpu_scores[:n], dtype=np.float32)),
                     list_digest=digest(np.asarray(gpu_list, dtype=np.int32)))


# ---------------------------------------------------------------------------
# Negative controls: each must make the row's check fail.
# ---------------------------------------------------------------------------


def control_replace_best_unselected(gpu_list, gpu_scores, n, k):
    """Replace one selected position by the best unselected one (list re-sorted)."""
    lst = np.asarray(gpu_list, dtype=np.int32).copy()
    sel = [int(x) for x in lst if x >= 0]
    if len(sel) == 0 or len(sel) >= n:
        return None
    chosen = set(sel)
    x = np.asarray(gpu_scores[:n], dtype=np.float64)
    order = np.lexsort((np.arange(n), -x))
    best_un = next(int(p) for p in order if int(p) not in chosen)
    sel[len(sel) // 2] = best_un
    sel.sort()
    lst[: len(sel)] = sel
    return lst


def control_swap(gpu_list):
    lst = np.asarray(gpu_list, dtype=np.int32).copy()
    valid = int((lst >= 0).sum())
    if valid < 2:
        return None
    i, j = 0, valid - 1
    lst[i], lst[j] = lst[j], lst[i]
    return lst


def control_flip_score(gpu_scores, n):
    """Flip the top exponent bit of the largest-magnitude score."""
    s = np.asarray(gpu_scores[:n], dtype=np.float32).copy()
    if n == 0:
        return None
    i = int(np.argmax(np.abs(s)))
    u = s.view(np.uint32)
    u[i] ^= np.uint32(0x40000000)
    return s


def negative_controls_fail(gpu_scores, gpu_list, ref_scores, n, k) -> List[bool]:
    """For each applicable control, True when the tampered copy fails the checks."""
    results = []
    c1 = control_replace_best_unselected(gpu_list, gpu_scores, n, k)
    if c1 is not None:
        results.append(not list_exact(c1, gpu_scores[:n], n, k))
    c2 = control_swap(gpu_list)
    if c2 is not None:
        results.append(not list_exact(c2, gpu_scores[:n], n, k))
    c3 = control_flip_score(gpu_scores, n)
    if c3 is not None:
        results.append(not score_error(c3, ref_scores[:n])[1])
    return results
