"""Keys written in the same launch (idx_score_topk_append): every row's new key is
scored from its (codes, scale) pair and stored to the cache.  The cache slots the
launch writes are poisoned beforehand (NaN codes and scale), so a launch that read
them from the cache would produce NaN scores and fail the bound."""
import dataclasses

import numpy as np
import pytest
import torch

import key_scoring_exact_amd as idx
from oracle import indexer as O
from workloads import make_problem
from workloads.synth import quantize_keys

from .gpu_helpers import check_against_oracle, device_problem

pytestmark = pytest.mark.gpu


def new_keys(prob, seed, skip=()):
    rng = np.random.default_rng(seed)
    codes, scales = quantize_keys(rng.standard_normal((prob.rows, prob.dim), dtype=np.float32) * np.float32(3.0))
    pos = prob.n_keys.astype(np.int32) - 1                   # each row's own last key
    for r in skip:
        pos[r] = -1
    return codes.astype(np.uint8), scales.astype(np.float32), pos


def poisoned(prob, pos):
    kc = prob.k_cache.copy().reshape(-1, prob.dim)
    ks = prob.k_scale.copy().reshape(-1)
    for r in range(prob.rows):
        if pos[r] >= 0:
            slot = int(prob.page_table[r][pos[r] // prob.page_size]) * prob.page_size + pos[r] % prob.page_size
            kc[slot] = 0x7F                                  # E4M3FN NaN
            ks[slot] = np.nan
    return dataclasses.replace(prob, k_cache=kc.reshape(prob.k_cache.shape), k_scale=ks.reshape(prob.k_scale.shape))


@pytest.mark.parametrize("contexts,rows,skip", [([3000], [4], ()), ([131072], [4], (1,)), ([9000], [8], ()),
                                                 ([40000], [8], (0, 5)), ([700, 30000, 5000], [2, 8, 3], (2,))])
def test_append_keys(contexts, rows, skip):
    prob = make_problem(contexts, rows, seed=9700 + sum(contexts) + sum(rows), name=f"append{contexts}x{rows}")
    codes, scales, pos = new_keys(prob, 5 + sum(rows), skip)
    bad = poisoned(prob, pos)
    print(f"case append {contexts} {rows} skip={skip}", flush=True)
    dp = device_problem(bad)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    cd = torch.from_numpy(codes).cuda()
    sd = torch.from_numpy(scales).cuda()
    pd = torch.from_numpy(pos).cuda()
    sc, ls = idx.score_topk_append(dp, prob.k, ws, cd, sd, pd)
    code, detail = idx.device_status(ws)
    assert code == 0, hex(detail)
    want = O.with_new_keys(prob, codes, scales, pos)
    # the cache now holds the new keys (and is otherwise unchanged)
    assert np.array_equal(dp.k_cache.cpu().numpy().view(np.uint8), want.k_cache)
    assert np.array_equal(dp.k_scale.cpu().numpy(), want.k_scale)
    s = sc.cpu().numpy()
    res = dict(scores=s, lists=ls.cpu().numpy(), scores_only=s, lists_topk=ls.cpu().numpy(), code=0, detail=0)
    check_against_oracle(want, res)
    # and a plain call on the written cache gives the same scores, bit for bit
    sc2, ls2 = idx.score_topk(dp, prob.k, ws)
    for r in range(prob.rows):
        n = int(prob.n_keys[r])
        assert np.array_equal(sc2.cpu().numpy()[r, :n].view(np.uint32), s[r, :n].view(np.uint32)), r
    assert np.array_equal(ls2.cpu().numpy(), ls.cpu().numpy())


@pytest.mark.parametrize("case", range(8))
def test_append_random(case):
    """Seeded random chains with keys written in the launch: 1-2 requests of 1-8 rows over
    100-250,000 keys, every cache kind, k from 1 to 2048, a random set of rows without a
    new key."""
    rng = np.random.default_rng(13579 + case)
    nreq = int(rng.integers(1, 3))
    contexts = [int(rng.integers(100, 250001)) for _ in range(nreq)]
    rows = [int(rng.integers(1, 9)) for _ in range(nreq)]
    k = int(rng.choice([1, 64, 300, 1024, 2048]))
    keys = str(rng.choice(["normal", "ties", "zeros", "recent"]))
    prob = make_problem(contexts, rows, seed=80000 + case, k=k, keys=keys, recent=int(rng.integers(64, 8192)),
                        name=f"append_random{case}")
    skip = tuple(int(r) for r in np.nonzero(rng.random(prob.rows) < 0.25)[0])
    codes, scales, pos = new_keys(prob, 90000 + case, skip)
    bad = poisoned(prob, pos)
    print(f"case append_random{case} contexts={contexts} rows={rows} k={k} keys={keys} skip={skip}", flush=True)
    dp = device_problem(bad)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    sc, ls = idx.score_topk_append(dp, prob.k, ws, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                   torch.from_numpy(pos).cuda())
    code, detail = idx.device_status(ws)
    assert code == 0, hex(detail)
    want = O.with_new_keys(prob, codes, scales, pos)
    assert np.array_equal(dp.k_cache.cpu().numpy().view(np.uint8), want.k_cache)
    assert np.array_equal(dp.k_scale.cpu().numpy(), want.k_scale)
    s_ = sc.cpu().numpy()
    check_against_oracle(want, dict(scores=s_, lists=ls.cpu().numpy(), scores_only=s_, lists_topk=ls.cpu().numpy(),
                                    code=0, detail=0))


def test_append_bad_position_reported():
    """A position at or past the row's key count is reported (IDX_DERR_NKEYS) and not written."""
    prob = make_problem([3000], [4], seed=31, name="append_bad")
    codes, scales, pos = new_keys(prob, 3)
    pos[2] = int(prob.n_keys[2])                              # one past what row 2 sees
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    idx.score_topk_append(dp, prob.k, ws, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                          torch.from_numpy(pos).cuda())
    code, detail = idx.device_status(ws)
    assert code == idx._lib.IDX_EDEVICE and detail & idx._lib.IDX_DERR_NKEYS


def test_append_bad_position_dropped_by_every_group():
    """An 8-row chain (two row groups).  Row 1 (first group) brings a key at a position
    past its own key count that only the second group's rows see; rows 4-7 write no key.
    The first group reports and drops it; the second group must drop it too and score
    the key the cache holds there.  Every row then matches the oracle on the cache with
    the valid keys written, and that slot is left as it was."""
    prob = make_problem([9000], [8], seed=9711, name="append_bad8")
    codes, scales, pos = new_keys(prob, 17, skip=(4, 5, 6, 7))
    pos[1] = int(prob.n_keys[1]) + 2                          # seen by rows 4..7 only
    assert pos[1] >= prob.n_keys[3] and pos[1] < prob.n_keys[4]
    good = pos.copy()
    good[1] = -1
    bad = poisoned(prob, good)                                 # the valid keys' slots only
    print(f"case append bad pos {int(pos[1])}", flush=True)
    dp = device_problem(bad)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    sc, ls = idx.score_topk_append(dp, prob.k, ws, torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                                   torch.from_numpy(pos).cuda())
    code, detail = idx.device_status(ws)
    assert code == idx._lib.IDX_EDEVICE and detail == idx._lib.IDX_DERR_NKEYS, hex(detail)
    want = O.with_new_keys(prob, codes, scales, good)
    assert np.array_equal(dp.k_cache.cpu().numpy().view(np.uint8), want.k_cache)
    assert np.array_equal(dp.k_scale.cpu().numpy(), want.k_scale)
    s = sc.cpu().numpy()
    res = dict(scores=s, lists=ls.cpu().numpy(), scores_only=s, lists_topk=ls.cpu().numpy(), code=0, detail=0)
    check_against_oracle(want, res)
