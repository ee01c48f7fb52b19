"""Pins of the CPU oracle to things other than itself.

The pages print no worked example, so each part of the oracle is pinned by a
library routine, a hand-derived closed form, brute force on tiny inputs or an
invariant of the score definition (GLM-5.3 indexer page, Modifications item
0: f64 score reference; exactness by score descending, then position).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import indexer as O

E4M3 = {  # hand-derived from the OCP E4M3FN definition (bias 7, 3 mantissa bits)
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
    0x38: 1.0, 0x39: 1.125, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0,
    0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0,
}


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = O.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_decode_spot_values():
    for c, v in E4M3.items():
        got = float(O.decode_e4m3fn(np.array([c], dtype=np.uint8))[0])
        assert got == v and np.signbit(got) == np.signbit(v), hex(c)
    assert np.isnan(O.decode_e4m3fn(np.array([0x7F, 0xFF], dtype=np.uint8))).all()
    finite = O.E4M3FN[~np.isnan(O.E4M3FN)]
    assert finite.max() == 448.0 and len(finite) == 254


def test_bf16_decode_matches_torch_all_codes():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    got = O.decode_bf16(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert O.decode_bf16(np.array([0x3F80, 0xC000, 0x3E00], dtype=np.uint16)).tolist() == [1.0, -2.0, 0.125]


def _bf16(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _e4m3(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_hand_example_closed_form():
    """H=2 heads, D=3, page size 2, three keys on a permuted two-page pool.

    q = [[1, 2, -1], [0.5, -1, 3]], w = [2, -0.5]
    keys (logical order) k0 = [1, .5, 2] s=1; k1 = [-1, 1, 1] s=.5; k2 = [0, 0, -2] s=2
    p=0: head0 1*(1+1-2)=0 -> 0; head1 1*(.5-.5+6)=6 -> 6;   score = 2*0 - .5*6 = -3
    p=1: head0 .5*(-1+2-1)=0 -> 0; head1 .5*(-.5-1+3)=.75;  score = -.375
    p=2: head0 2*(0+0+2)=4 -> 4;   head1 2*(0+0-6)=-12 -> 0; score = 8
    """
    q = _bf16([[1, 2, -1], [0.5, -1, 3]])
    w = _bf16([2, -0.5])
    keys = _e4m3([[1, 0.5, 2], [-1, 1, 1], [0, 0, -2], [0, 0, 0]])
    scales = np.array([1.0, 0.5, 2.0, 0.0], dtype=np.float32)
    # logical page 0 (positions 0,1) -> physical page 1; logical page 1 (2,3) -> physical 0
    cache = np.zeros((2, 2, 3), dtype=np.uint8)
    kscale = np.zeros((2, 2), dtype=np.float32)
    cache[1] = keys[0:2]; kscale[1] = scales[0:2]
    cache[0] = keys[2:4]; kscale[0] = scales[2:4]
    v = O.row_scores(q, w, cache, kscale, np.array([1, 0], dtype=np.int32), 3)
    assert v.tolist() == [-3.0, -0.375, 8.0]
    assert O.select(v, 3, 2).tolist() == [1, 2]
    assert O.select(v, 3, 1).tolist() == [2]
    assert O.select(v, 3, 4).tolist() == [0, 1, 2, -1]


def test_single_head_single_dim_closed_form():
    """H = D = 1: score = w * max(s*q*k, 0)."""
    rng = np.random.default_rng(5)
    for _ in range(50):
        qv, wv, kv = rng.choice([-2, -1, -0.5, 0.5, 1, 1.5, 3], size=3)
        s = float(rng.choice([0.0, 0.25, 1.0, 2.0]))
        v = O.row_scores(_bf16([[qv]]), _bf16([wv]), _e4m3([[kv]]).reshape(1, 1, 1),
                         np.array([[s]], dtype=np.float32), np.array([0], dtype=np.int32), 1)
        assert v[0] == wv * max(s * qv * kv, 0.0)


def test_gather_reads_each_position_from_its_page():
    """Each logical position carries a unique scale; with q = k = w = 1 (H = D = 1)
    the score of position p is that scale, wherever the page table puts it."""
    rng = np.random.default_rng(11)
    page, n = 4, 37
    npages = (n + page - 1) // page + 3          # spare pages in the pool
    perm = rng.permutation(npages)[: (n + page - 1) // page]
    cache = np.full((npages, page, 1), 0x38, dtype=np.uint8)   # every key value 1.0
    kscale = np.full((npages, page), 1000.0, dtype=np.float32)  # untouched slots: 1000
    for p in range(n):
        kscale[perm[p // page], p % page] = p + 1
    v = O.row_scores(_bf16([[1.0]]), _bf16([1.0]), cache, kscale, perm.astype(np.int32), n)
    assert v.tolist() == [float(p + 1) for p in range(n)]


def _tiny_problem(rng, H, D, page, n, npages):
    q = _bf16(rng.choice([-3, -1.5, -1, -0.25, 0, 0.5, 1, 2], size=(H, D)))
    w = _bf16(rng.choice([-1, -0.5, 0.25, 0.5, 1], size=(H,)))
    cache = rng.integers(0, 256, size=(npages, page, D)).astype(np.uint8)
    cache[(cache & 0x7F) == 0x7F] = 0x38                        # no NaN codes
    kscale = rng.choice([0.0, 0.125, 0.5, 1.0, 3.0], size=(npages, page)).astype(np.float32)
    table = rng.permutation(npages)[: (n + page - 1) // page].astype(np.int32)
    return q, w, cache, kscale, table


def test_exact_rational_scores_on_tiny_inputs():
    """All inputs are dyadic rationals, so the score is an exact Fraction; the
    f64 oracle must agree to 1e-12 relative to the row's largest |score|."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        H, D, page, n = 3, 4, 4, 10
        q, w, cache, kscale, table = _tiny_problem(rng, H, D, page, n, 4)
        v = O.row_scores(q, w, cache, kscale, table, n)
        Q = [[Fraction(float(x)) for x in row] for row in O.decode_bf16(q)]
        W = [Fraction(float(x)) for x in O.decode_bf16(w)]
        exact = []
        for p in range(n):
            slot = cache[table[p // page], p % page]
            K = [Fraction(float(x)) for x in O.decode_e4m3fn(slot)]
            s = Fraction(float(kscale[table[p // page], p % page]))
            tot = Fraction(0)
            for h in range(H):
                lg = s * sum(Q[h][d] * K[d] for d in range(D))
                tot += W[h] * max(lg, Fraction(0))
            exact.append(tot)
        m = max(abs(float(e)) for e in exact) or 1.0
        assert max(abs(v[p] - float(exact[p])) for p in range(n)) <= 1e-12 * m


def test_score_invariants():
    rng = np.random.default_rng(9)
    H, D, page, n = 8, 16, 8, 40
    q, w, cache, kscale, table = _tiny_problem(rng, H, D, page, n, 6)
    v = O.row_scores(q, w, cache, kscale, table, n)
    # a different physical layout of the same logical keys gives identical scores
    npages = cache.shape[0]
    perm2 = rng.permutation(npages).astype(np.int32)
    cache2 = np.zeros_like(cache); kscale2 = np.zeros_like(kscale)
    for j, phys in enumerate(table):
        cache2[perm2[j]] = cache[phys]; kscale2[perm2[j]] = kscale[phys]
    assert np.array_equal(O.row_scores(q, w, cache2, kscale2, perm2[: len(table)], n), v)
    # scaling one key's scale by 2^j scales its score by exactly 2^j, nothing else moves
    p = 13
    k2 = kscale.copy(); k2[table[p // page], p % page] *= 8
    v2 = O.row_scores(q, w, cache, k2, table, n)
    assert v2[p] == 8 * v[p] and np.array_equal(np.delete(v2, p), np.delete(v, p))
    # negating the head weights negates every score
    wn = (w ^ np.uint16(0x8000)).astype(np.uint16)
    assert np.array_equal(O.row_scores(q, wn, cache, kscale, table, n), -v)
    # doubling q doubles every score (ReLU is positively homogeneous)
    q2 = _bf16(2 * O.decode_bf16(q))
    assert np.array_equal(O.row_scores(q2, w, cache, kscale, table, n), 2 * v)
    # all-zero keys and zero scales give exactly zero
    assert np.all(O.row_scores(q, w, np.zeros_like(cache), kscale, table, n) == 0)
    assert np.all(O.row_scores(q, w, cache, np.zeros_like(kscale), table, n) == 0)
    # a head whose logits are all negative contributes nothing: append head -q_0
    # with weight 5 where head 0 ... use keys with one nonzero coordinate
    cache1 = np.zeros_like(cache); cache1[..., 0] = 0x38          # every key = e_0
    qa = np.zeros((2, D), dtype=np.uint16)
    qa[0] = _bf16(np.r_[[1.0], np.zeros(D - 1)]); qa[1] = _bf16(np.r_[[-1.0], np.zeros(D - 1)])
    va = O.row_scores(qa, _bf16([1.0, 5.0]), cache1, np.ones_like(kscale), table, n)
    assert np.all(va == 1.0)
    # duplicate keys get equal scores
    cd = cache.copy(); cd[table[1], 3] = cd[table[0], 2]
    kd = kscale.copy(); kd[table[1], 3] = kd[table[0], 2]
    vd = O.row_scores(q, w, cd, kd, table, n)
    assert vd[page + 3] == vd[2]


def _brute_select(v, n, k):
    """The unique k-subset S with every s in S beating every u outside it:
    v[s] > v[u], or v[s] == v[u] and s < u."""
    if n <= k:
        return list(range(n)) + [-1] * (k - n)
    found = []
    for S in itertools.combinations(range(n), k):
        Sset = set(S)
        if all((v[s] > v[u]) or (v[s] == v[u] and s < u) for s in S for u in range(n) if u not in Sset):
            found.append(list(S))
    assert len(found) == 1
    return found[0]


def test_select_brute_force_tiny():
    rng = np.random.default_rng(17)
    for trial in range(120):
        n = int(rng.integers(0, 10))
        k = int(rng.integers(1, 12))
        v = rng.choice([-1.0, -0.0, 0.0, 0.5, 0.5, 2.0, 3.0], size=n)
        assert O.select(v, n, k).tolist() == _brute_select(v.tolist(), n, k), (v, n, k)


def test_select_special_cases():
    assert O.select(np.array([]), 0, 4).tolist() == [-1, -1, -1, -1]
    assert O.select(np.array([5.0, 1.0, 3.0]), 3, 5).tolist() == [0, 1, 2, -1, -1]
    assert O.select(np.array([5.0, 1.0, 3.0]), 3, 3).tolist() == [0, 1, 2]
    assert O.select(np.full(100, 7.0), 100, 10).tolist() == list(range(10))
    # -0 ties +0: the lower position wins, whichever sign it carries
    assert O.select(np.array([-0.0, 0.0, -1.0]), 3, 1).tolist() == [0]
    assert O.select(np.array([1.0, -0.0, 0.0, 0.0]), 4, 2).tolist() == [0, 1]
    # emission is ascending even when the best key is last
    assert O.select(np.array([1.0, 2.0, 9.0, 0.0, 8.0]), 5, 3).tolist() == [1, 2, 4]
    with pytest.raises(ValueError):
        O.select(np.array([np.nan, 1.0]), 2, 1)


def test_list_slots_identity_and_permutation():
    """Slots of a list: with an identity page table they are the positions; with a
    permuted table position p maps into page perm[p // 64] at slot p % 64; -1 stays."""
    from workloads import make_problem
    prob = make_problem([300], [2], seed=11, k=8, name="slots")
    lists = np.array([[0, 1, 63, 64, 65, 299, -1, -1], [5, 70, 128, 200, 250, 296, 297, 298]])
    ident = prob.page_table.copy()
    ident[:] = np.arange(ident.shape[1])
    prob.page_table = ident
    assert np.array_equal(O.list_slots(prob, lists), lists)
    perm = np.array([3, 0, 4, 1, 2], dtype=np.int32)
    prob.page_table = np.tile(perm, (2, 1))
    got = O.list_slots(prob, lists)
    assert got[0, 0] == 3 * 64 and got[0, 2] == 3 * 64 + 63 and got[0, 3] == 0 and got[0, 5] == 2 * 64 + 43
    assert got[0, 6] == -1 and got[1, 2] == 4 * 64


def _hand_problem():
    """Three rows in two requests over a pool of four pages of two keys (D = 3, H = 1):
    rows 0 and 1 (request 0) map logical pages 0, 1 to physical pages 2, 0; row 2
    (request 1) maps its one logical page to physical page 1.  Page 3 is spare."""
    from workloads.synth import Problem
    kc = np.zeros((4, 2, 3), dtype=np.uint8)
    kc[...] = np.arange(24, dtype=np.uint8).reshape(4, 2, 3)   # distinct finite codes
    ks = (np.arange(8, dtype=np.float32).reshape(4, 2) + 1) / 4
    pt = np.array([[2, 0], [2, 0], [1, 1]], dtype=np.int32)
    return Problem(name="hand", q=_bf16(np.ones((3, 1, 3))), w=_bf16(np.ones((3, 1))), k_cache=kc, k_scale=ks,
                   page_table=pt, n_keys=np.array([4, 4, 2], dtype=np.int32),
                   req_indptr=np.array([0, 2, 3], dtype=np.int32), k=2, seed=0, heads=1, dim=3, page_size=2)


def test_with_new_keys_hand_worked():
    """Row 0 writes logical position 3: logical page 1 of its table is physical page 0,
    so flat slot 0 * 2 + 1 = 1.  Row 1 writes nothing (pos = -1).  Row 2 writes logical
    position 0 through its own table: physical page 1, flat slot 2.  Nothing else
    changes, and the inputs are left as they were."""
    prob = _hand_problem()
    kc0, ks0, pt0 = prob.k_cache.copy(), prob.k_scale.copy(), prob.page_table.copy()
    codes = np.array([[0x38, 0x40, 0x30], [0x01, 0x02, 0x03], [0xB8, 0x48, 0x00]], dtype=np.uint8)
    scales = np.array([0.5, 9.0, 2.0], dtype=np.float32)
    pos = np.array([3, -1, 0], dtype=np.int32)
    out = O.with_new_keys(prob, codes, scales, pos)
    flat_c = out.k_cache.reshape(-1, 3)
    flat_s = out.k_scale.reshape(-1)
    want_c = kc0.reshape(-1, 3).copy()
    want_s = ks0.reshape(-1).copy()
    want_c[1], want_s[1] = codes[0], 0.5
    want_c[2], want_s[2] = codes[2], 2.0
    assert np.array_equal(flat_c, want_c) and np.array_equal(flat_s, want_s)
    assert out.k_cache.shape == kc0.shape and out.k_scale.shape == ks0.shape
    # the input problem is unchanged
    assert np.array_equal(prob.k_cache, kc0) and np.array_equal(prob.k_scale, ks0)
    assert np.array_equal(prob.page_table, pt0)
    # a slot written from row 0's page-table row for row 2 (slot 4) or from the
    # logical position taken as a flat slot (slot 3 for row 0) stays untouched
    assert np.array_equal(flat_c[3], kc0.reshape(-1, 3)[3]) and np.array_equal(flat_c[4], kc0.reshape(-1, 3)[4])


def test_with_new_keys_scores_the_written_key():
    """Invariant: after the write, the score a row gives its written position equals
    (to f64 rounding) the score of a one-key cache holding just that key (codes,
    scale), and every other position of every row keeps its score bit for bit."""
    from workloads import make_problem
    from workloads.synth import quantize_keys
    prob = make_problem([300, 150], [3, 2], seed=23, k=8, name="nk")
    rng = np.random.default_rng(4)
    codes, scales = quantize_keys(rng.standard_normal((prob.rows, prob.dim), dtype=np.float32))
    pos = np.array([10, -1, 297, 0, 148], dtype=np.int32)
    before = O.scores(prob)
    after = O.scores(O.with_new_keys(prob, codes, scales, pos))
    for r in range(prob.rows):
        n = int(prob.n_keys[r])
        # positions a row's request writes (this row's and its request mates')
        a, b = [(s, e) for s, e in zip(prob.req_indptr[:-1], prob.req_indptr[1:]) if s <= r < e][0]
        written = {int(pos[j]) for j in range(a, b) if pos[j] >= 0}
        for p in range(n):
            if p not in written:
                assert after[r][p] == before[r][p], (r, p)
        for j in range(a, b):
            p = int(pos[j])
            if 0 <= p < n:
                one = O.row_scores(prob.q[r], prob.w[r], codes[j].reshape(1, 1, -1),
                                   np.array([[scales[j]]], dtype=np.float32), np.array([0], dtype=np.int32), 1)
                # equal up to f64 summation order (a misplaced key differs at O(1))
                assert abs(after[r][p] - one[0]) <= 1e-12 * max(1.0, abs(one[0])), (r, j, p)
