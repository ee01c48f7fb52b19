"""CPU oracle for the sparse-attention indexer: exact key scores and exact top-k.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module; only tests, the smoke check and the benchmark's CPU
baseline use it.  It shares no code with the GPU library.

What is computed (per row r with n = n_keys[r] keys):

* The GLM-5.3 indexer page (sgl-amd-mono-upstream pull request 18),
  Modifications item 0, checks each launch's scores against an f64
  reference built from the launch's bf16 index query, its head weights and
  the row's keys.  The score of logical position p is

      score[r, p] = sum_h w[r, h] * ReLU( s[p] * sum_d q[r, h, d] * k8[p, d] )

  with k8 the key's OCP FP8-E4M3FN value and s its per-key f32 scale.  The
  page states no equation; this is the plain reading used throughout (the
  head-weighted sum of ReLU'd, key-scaled dot products).
* Keys are found through the paged cache: position p of row r lives in
  physical page page_table[r][p // page_size], slot p % page_size.  Each row
  uses its own page-table row (the same page, item 0's test fix: a page-table
  row per step row).
* The same item defines exactness by score descending, then position: the
  top-k set is the first k positions in that order.  The list is emitted in
  ascending position order; a row with n <= k selects all n positions and
  pads with -1.

Everything is evaluated in float64 (bf16 and E4M3 values, scales and
products are exact in f64; only the summations round, far below 1e-4 of the
row's largest score); the dot products use one fixed summation order for
every position.  The selection is a full sort by (-score, position).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Decoders, written from the number formats' definitions.
# ---------------------------------------------------------------------------


def _e4m3fn_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3FN code: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal, (m/8) * 2^-6; otherwise (1 + m/8) * 2^(e-7).
    There are no infinities; S.1111.111 is NaN; the largest finite value is 448.
    """
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if (c >> 7) & 1 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3FN = _e4m3fn_table()


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """FP8 E4M3FN codes (uint8) -> float64."""
    return E4M3FN[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the upper half of an IEEE binary32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Scoring
# ---------------------------------------------------------------------------


def row_slots(page_table_row: np.ndarray, n: int, page_size: int) -> np.ndarray:
    """Flat cache slot of each logical position 0..n-1 of one row."""
    p = np.arange(n, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[p // page_size]
    return pages * page_size + p % page_size


def row_scores(q_bits: np.ndarray, w_bits: np.ndarray, k_cache: np.ndarray,
               k_scale: np.ndarray, page_table_row: np.ndarray, n: int) -> np.ndarray:
    """f64 scores of positions 0..n-1 for one row.

    q_bits: uint16 [H, D]; w_bits: uint16 [H]; k_cache: uint8 [pages, page, D];
    k_scale: float32 [pages, page].
    """
    page_size = k_cache.shape[1]
    dim = k_cache.shape[2]
    slots = row_slots(page_table_row, n, page_size)
    K = decode_e4m3fn(k_cache.reshape(-1, dim)[slots])           # [n, D]
    S = k_scale.reshape(-1)[slots].astype(np.float64)           # [n]
    if np.isnan(K).any() or not np.isfinite(S).all() or (S < 0).any():
        raise ValueError("key cache holds NaN codes or invalid scales")
    Q = decode_bf16(q_bits)                                     # [H, D]
    W = decode_bf16(w_bits)                                     # [H]
    # einsum without BLAS sums over d (and below over h) in one fixed order for
    # every position, so bit-identical keys get bit-identical scores (a blocked
    # GEMM may round edge columns differently, which would break exact ties).
    dots = np.einsum("hd,nd->hn", Q, K, optimize=False)        # [H, n]
    logits = S[None, :] * dots
    return np.einsum("h,hn->n", W, np.maximum(logits, 0.0), optimize=False)  # [n]


def scores(problem) -> list:
    """Per-row f64 score vectors for every row of a workloads.Problem."""
    out = []
    for r in range(problem.rows):
        n = int(problem.n_keys[r])
        out.append(row_scores(problem.q[r], problem.w[r], problem.k_cache,
                              problem.k_scale, problem.page_table[r], n))
    return out


# ---------------------------------------------------------------------------
# Selection
# ---------------------------------------------------------------------------


def select(v: np.ndarray, n: int, k: int) -> np.ndarray:
    """Exact top-k positions of v[0:n] by (score desc, position asc), emitted ascending.

    Scores compare as real numbers (so -0 equals +0 and the lower position
    wins the tie).  Returns int32 [k], padded with -1 when n < k.
    """
    out = np.full(k, -1, dtype=np.int32)
    if n <= k:
        out[:n] = np.arange(n, dtype=np.int32)
        return out
    x = np.asarray(v[:n], dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN score")
    pos = np.arange(n, dtype=np.int64)
    order = np.lexsort((pos, -x))            # primary key -score, then position
    out[:] = np.sort(order[:k]).astype(np.int32)
    return out


def topk(problem, row_scores_list=None) -> np.ndarray:
    """[rows, k] int32 lists from oracle scores (or from given per-row scores)."""
    vs = scores(problem) if row_scores_list is None else row_scores_list
    out = np.empty((problem.rows, problem.k), dtype=np.int32)
    for r in range(problem.rows):
        out[r] = select(vs[r], int(problem.n_keys[r]), problem.k)
    return out


def list_slots(problem, lists: np.ndarray) -> np.ndarray:
    """Each list entry as its physical cache slot, through the row's own page-table row
    (the same gather as the scoring: position p lives in page page_table[r][p // page]
    at slot p % page); -1 padding stays -1."""
    lists = np.asarray(lists, dtype=np.int64)
    out = np.full(lists.shape, -1, dtype=np.int64)
    for r in range(lists.shape[0]):
        p = lists[r]
        m = p >= 0
        out[r, m] = problem.page_table[r][p[m] // problem.page_size].astype(np.int64) * problem.page_size + \
            p[m] % problem.page_size
    return out


def with_new_keys(problem, codes: np.ndarray, scales: np.ndarray, pos: np.ndarray):
    """The problem with each row's new key written into its cache: row r's codes[r] and
    scales[r] at logical position pos[r] (-1: none), physical slot page_table[r][pos //
    page] * page + pos % page.  Returns a copy; the input is unchanged."""
    import copy
    out = copy.copy(problem)
    kc = problem.k_cache.copy().reshape(-1, problem.dim)
    ks = problem.k_scale.copy().reshape(-1)
    for r in range(problem.rows):
        p = int(pos[r])
        if p < 0:
            continue
        slot = int(problem.page_table[r][p // problem.page_size]) * problem.page_size + p % problem.page_size
        kc[slot] = codes[r]
        ks[slot] = scales[r]
    out.k_cache = kc.reshape(problem.k_cache.shape)
    out.k_scale = ks.reshape(problem.k_scale.shape)
    return out
