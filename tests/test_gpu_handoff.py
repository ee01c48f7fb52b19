"""Tagged hand-off of the selected slots (idx_score_topk_tagged): every list entry's cache
slot is written as one 64-bit word tag << 32 | slot, the form a consumer polls without a
ready flag (the GLM-5.3-Flash hand-offs page, Modifications item 3).  Checked against the
oracle's slot map of the GPU's lists, and against the untagged entry points."""
import numpy as np
import pytest
import torch

import key_scoring_exact_amd as idx
from oracle import indexer as O
from workloads import make_problem

from .gpu_helpers import check_against_oracle, device_problem

pytestmark = pytest.mark.gpu


def ready(words: np.ndarray, tag: int) -> np.ndarray:
    """The consumer's test of a word: its high half carries this call's tag."""
    return (words.view(np.uint64) >> np.uint64(32)) == np.uint64(tag)


def slots_of(words: np.ndarray) -> np.ndarray:
    return (words.view(np.uint64) & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.int32).astype(np.int64)


@pytest.mark.parametrize("contexts,rows", [([3000], [4]), ([131072], [4]), ([1500, 40000, 9000], [2, 3, 8])])
def test_tagged_slots(contexts, rows):
    prob = make_problem(contexts, rows, seed=9300 + sum(contexts), name=f"tagged{contexts}")
    print(f"case tagged {contexts} {rows}", flush=True)
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    stale = torch.full((prob.rows, prob.k), -1, dtype=torch.int64, device="cuda")     # every word "not ready"
    tag = 0x5EED0001
    sc, ls, tg = idx.score_topk_tagged(dp, prob.k, ws, tag, tagged=stale)
    sc2, ls2, sl2 = idx.score_topk_slots(dp, prob.k, ws)
    assert idx.device_status(ws)[0] == 0
    words, ls = tg.cpu().numpy(), ls.cpu().numpy()
    assert ready(words, tag).all()
    assert np.array_equal(slots_of(words), O.list_slots(prob, ls))
    assert np.array_equal(slots_of(words), sl2.cpu().numpy())
    assert np.array_equal(ls, ls2.cpu().numpy())
    res = dict(scores=sc.cpu().numpy(), lists=ls, scores_only=sc.cpu().numpy(), lists_topk=ls, code=0, detail=0)
    check_against_oracle(prob, res)
    # a word left from an earlier call (an older tag) is not ready under the new tag
    old = words.copy().view(np.uint64)
    old[0, 0] = (np.uint64(tag - 1) << np.uint64(32)) | (old[0, 0] & np.uint64(0xFFFFFFFF))
    assert not ready(old.view(np.int64), tag)[0, 0]
    # the next call's tag rewrites every word
    _, _, tg2 = idx.score_topk_tagged(dp, prob.k, ws, tag + 1, tagged=tg)
    w2 = tg2.cpu().numpy()
    assert ready(w2, tag + 1).all() and np.array_equal(slots_of(w2), slots_of(words))


@pytest.mark.parametrize("case", range(6))
def test_tagged_slots_random(case):
    """Seeded random problems (1-3 requests of 1-8 rows over 1-200,000 keys, every cache
    kind, k from 1 to 2048, spare pool pages) through two tagged calls in a row: every
    word ready under its call's tag, the slots equal to the oracle's map of the list."""
    rng = np.random.default_rng(11223 + case)
    nreq = int(rng.integers(1, 4))
    contexts = [int(rng.integers(1, 200001)) for _ in range(nreq)]
    rows = [int(rng.integers(1, 9)) for _ in range(nreq)]
    k = int(rng.choice([1, 64, 300, 1024, 2048]))
    keys = str(rng.choice(["normal", "ties", "zeros", "recent"]))
    prob = make_problem(contexts, rows, seed=30000 + case, k=k, keys=keys, chain=bool(rng.random() < 0.6),
                        pad_pages=int(rng.integers(0, 5)), name=f"tagged_random{case}")
    print(f"case {prob.name} contexts={contexts} rows={rows} k={k} keys={keys}", flush=True)
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    words = torch.full((prob.rows, prob.k), -1, dtype=torch.int64, device="cuda")
    for tag in (0x7A650000 + case, 0x7A650100 + case):
        sc, ls, tg = idx.score_topk_tagged(dp, prob.k, ws, tag, tagged=words)
        assert idx.device_status(ws)[0] == 0
        w, l_ = tg.cpu().numpy(), ls.cpu().numpy()
        assert ready(w, tag).all()
        assert np.array_equal(slots_of(w), O.list_slots(prob, l_))
        res = dict(scores=sc.cpu().numpy(), lists=l_, scores_only=sc.cpu().numpy(), lists_topk=l_, code=0, detail=0)
        check_against_oracle(prob, res)

