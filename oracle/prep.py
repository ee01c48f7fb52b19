"""CPU oracle for index-query preparation: RoPE, then the orthonormal Hadamard transform.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute
this module; only tests use it.  It shares no code with the GPU library.

What is computed (the GLM-5.3 indexer page, Modifications item 2, on preparing the
query once a row: each row's index query gets its rotary embedding and the Hadamard
transform a single time and is stored as bf16; Modifications item 0 derives its f64
score reference from that prepared query, whose arithmetic is f32 with one final
rounding to bf16).  The page gives no
formula; the plain reading taken here, per row r and head h, with x = q_pre[r, h, :]:

* RoPE on the first ``rope_dim`` dimensions (rope_dim even), with the caller's
  per-row rotation table (cos[r, i], sin[r, i]) for i < rope_dim / 2.  Pair i is
  (i, i + rope_dim / 2) in the half-split layout, (2 i, 2 i + 1) interleaved; the pair
  (a, b) becomes (a cos - b sin, a sin + b cos).  Dimensions >= rope_dim pass through.
* Then y = H x / sqrt(D), H the Sylvester Hadamard matrix of order D (a power of two):
  H[i, j] = (-1) ** popcount(i & j).  H / sqrt(D) is orthonormal and symmetric, so the
  transform is its own inverse.

Everything is evaluated in float64; the published query is bf16, so comparisons are
made against the f64 value with a one-unit-in-the-last-place bound.
"""
from __future__ import annotations

import numpy as np

from .indexer import decode_bf16


def sylvester(d: int) -> np.ndarray:
    """The Sylvester Hadamard matrix of order d (a power of two), from its recursion
    H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    assert d >= 1 and d & (d - 1) == 0
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, rope_dim: int, interleaved: bool) -> np.ndarray:
    """RoPE of x [rows, heads, d] (f64) on its first rope_dim dims; cos, sin [rows, rope_dim / 2]."""
    y = np.array(x, dtype=np.float64, copy=True)
    half = rope_dim // 2
    if half == 0:
        return y
    c = np.asarray(cos, dtype=np.float64)[:, None, :half]
    s = np.asarray(sin, dtype=np.float64)[:, None, :half]
    if interleaved:
        a, b = x[..., 0:rope_dim:2], x[..., 1:rope_dim:2]
        y[..., 0:rope_dim:2] = a * c - b * s
        y[..., 1:rope_dim:2] = a * s + b * c
    else:
        a, b = x[..., :half], x[..., half:rope_dim]
        y[..., :half] = a * c - b * s
        y[..., half:rope_dim] = a * s + b * c
    return y


def hadamard(x: np.ndarray) -> np.ndarray:
    """x [..., d] -> x H / sqrt(d) in f64 (H symmetric)."""
    d = x.shape[-1]
    return np.asarray(x, dtype=np.float64) @ (sylvester(d) / np.sqrt(d))


def prep_query(q_pre_bits: np.ndarray, cos: np.ndarray, sin: np.ndarray, rope_dim: int,
               interleaved: bool = False) -> np.ndarray:
    """The prepared index query in f64 (before its bf16 rounding): [rows, heads, d]."""
    x = decode_bf16(q_pre_bits)
    return hadamard(rope(x, cos, sin, rope_dim, interleaved))


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """The spacing of bf16 values at |v| (8 significant bits; the smallest normal's
    spacing below it)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)
