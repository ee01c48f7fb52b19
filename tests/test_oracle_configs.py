"""Closed forms and invariants of the adversarial caches, the checker's negative
controls, and generator determinism (all CPU).

The caches are those of the GLM-5.3 indexer page's exact top-k check
(Modifications item 0): four keys repeated over every position (ties),
all-zero keys, and each row's last 4,096 keys scaled 8x (recent).
"""
import numpy as np
import pytest

from oracle import indexer as O
from oracle import check as C
from workloads import make_config, make_problem


def test_config_shapes():
    p = make_config("c3", scale_down=1)
    assert p.rows == 16 and p.num_req == 4 and p.num_pages == 24 + 128 + 512 + 2048
    assert p.n_keys.tolist() == [1497, 1498, 1499, 1500, 8189, 8190, 8191, 8192,
                                 32765, 32766, 32767, 32768, 131069, 131070, 131071, 131072]
    assert p.req_indptr.tolist() == [0, 4, 8, 12, 16]
    # pages of the requests are disjoint and together cover the pool
    used = np.concatenate([p.page_table[p.req_indptr[j], : (c + 63) // 64]
                           for j, c in enumerate([1500, 8192, 32768, 131072])])
    assert sorted(used.tolist()) == list(range(p.num_pages))
    p2 = make_config("c2")
    assert p2.n_keys.tolist() == [131069, 131070, 131071, 131072] and p2.num_pages == 2048
    assert sorted(p2.page_table[0].tolist()) == list(range(2048))
    assert p2.q.dtype == np.uint16 and p2.q.shape == (4, 64, 128)


def test_generator_deterministic():
    a = make_config("c1", scale_down=4)
    b = make_config("c1", scale_down=4)
    for f in ("q", "w", "k_cache", "k_scale", "page_table", "n_keys"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = make_problem([2048], [4], seed=99)
    assert not np.array_equal(a.q[:, :, :], c.q[: a.rows])


def test_quantisation_rule():
    p = make_config("c0")
    vals = O.decode_e4m3fn(p.k_cache)
    # every key's largest code is within one E4M3 step of 448 (amax / scale = 448 before rounding)
    top = np.abs(vals).max(axis=-1)
    assert np.all((top >= 416) & (top <= 448))
    assert np.all(p.k_scale > 0)


@pytest.mark.slow
def test_ties_cache_closed_form():
    p = make_config("c4a", scale_down=8)       # 16,384 keys, 4 rows
    vs = O.scores(p)
    lists = O.topk(p, vs)
    for r in range(p.rows):
        n = int(p.n_keys[r]); v = vs[r]
        # each residue class mod 4 holds one bit-identical key, so one score
        for j in range(4):
            assert np.all(v[j::4] == v[j])
        best = max(v[j] for j in range(4) if j < n)
        J = [j for j in range(4) if j < n and v[j] == best]
        want = [q for q in range(n) if q % 4 in J][: p.k]
        assert lists[r].tolist() == want


@pytest.mark.slow
def test_zero_cache_closed_form():
    p = make_config("c4b", scale_down=8)
    vs = O.scores(p)
    for r in range(p.rows):
        assert np.all(vs[r] == 0.0)
        assert O.select(vs[r], int(p.n_keys[r]), p.k).tolist() == list(range(p.k))
        e, ok = C.score_error(np.zeros(int(p.n_keys[r]), np.float32), vs[r])
        assert ok and e == 0.0
        e, ok = C.score_error(np.full(int(p.n_keys[r]), 1e-30, np.float32), vs[r])
        assert not ok


@pytest.mark.slow
def test_recent_cache_scales_exactly():
    p8 = make_config("c4c", scale_down=8)
    spec = dict(contexts=[131072 // 8], rows_per_req=[4], seed=42, keys="recent",
                recent=4096 // 8, recent_factor=1.0)
    p1 = make_problem(**spec)
    n0 = 131072 // 8
    lo = n0 - 4096 // 8
    assert np.array_equal(p8.k_cache, p1.k_cache)
    s8 = p8.k_scale.reshape(-1); s1 = p1.k_scale.reshape(-1)
    v8 = O.scores(p8); v1 = O.scores(p1)
    for r in range(p8.rows):
        n = int(p8.n_keys[r])
        assert np.array_equal(v8[r][lo:n], 8 * v1[r][lo:n])
        assert np.array_equal(v8[r][:lo], v1[r][:lo])
    slots = O.row_slots(p8.page_table[0], n0, 64)
    assert np.array_equal(s8[slots[lo:]], 8 * s1[slots[lo:]])


def test_checker_accepts_exact_and_rejects_controls():
    p = make_config("c1", scale_down=2)        # 4 rows of ~4,096 keys
    vs = O.scores(p)
    for r in range(p.rows):
        n = int(p.n_keys[r])
        gpu = vs[r].astype(np.float32)          # an f32-rounded "kernel" result
        lst = O.select(gpu.astype(np.float64), n, p.k)
        rep = C.check_row(r, gpu, lst, vs[r], n, p.k)
        assert rep.score_ok and rep.list_ok and rep.err_over_max < 1e-6
        assert all(C.negative_controls_fail(gpu, lst, vs[r], n, p.k))
        assert len(C.negative_controls_fail(gpu, lst, vs[r], n, p.k)) == 3
        # a list built from other scores is caught unless it happens to agree
        wrong = lst.copy(); wrong[0] = -1
        assert not C.list_exact(wrong, gpu, n, p.k)
    # "missed" counts reference top-k keys absent from the list
    n = int(p.n_keys[0])
    lst = O.select(vs[0], n, p.k)
    assert C.missed(lst, vs[0], n, p.k) == 0
    assert C.missed(C.control_replace_best_unselected(lst, vs[0], n, p.k), vs[0], n, p.k) == 1


def test_score_bound_uses_largest_magnitude():
    ref = np.array([-10.0, 1.0, 2.0])
    assert C.score_error(np.array([-10.0, 1.0, 2.0 + 9e-4], np.float32), ref)[1]
    assert not C.score_error(np.array([-10.0, 1.0, 2.0 + 2e-3], np.float32), ref)[1]
