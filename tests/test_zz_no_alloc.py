"""idx_score_topk_noalloc: the fused call with the library's static per-device scratch in
place of a workspace.  Two calls in a row, the second on a smaller problem, each against
idx_score_topk on the same inputs (scores bit for bit, lists exact) and against the
oracle (score bound, lists exact over the GPU's own scores); then six seeded random
problems back to back; and the host's refusal of a problem beyond the scratch."""
import numpy as np
import pytest
import torch

import key_scoring_exact_amd as idx
from key_scoring_exact_amd import _lib
from workloads import make_problem

from .gpu_helpers import check_against_oracle, device_problem

pytestmark = pytest.mark.gpu


def test_noalloc_matches_workspace_entry_point():
    probs = [make_problem([131072], [4], seed=9501, name="noalloc_big"),
             make_problem([700, 30000, 9000], [2, 3, 4], seed=9502, name="noalloc_small")]
    for prob in probs:
        print(f"case {prob.name} rows={prob.rows} max_keys={prob.max_keys}", flush=True)
        dp = device_problem(prob)
        ld = max(1, dp.max_keys)
        s_na = torch.full((prob.rows, ld), float("nan"), dtype=torch.float32, device="cuda")
        l_na = torch.full((prob.rows, prob.k), -7, dtype=torch.int32, device="cuda")
        idx.score_topk_noalloc(dp, prob.k, s_na, l_na)
        torch.cuda.synchronize()
        ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
        s_ws, l_ws = idx.score_topk(dp, prob.k, ws)
        assert idx.device_status(ws)[0] == 0
        a, b = s_na.cpu().numpy(), s_ws.cpu().numpy()
        for r in range(prob.rows):
            n = int(prob.n_keys[r])
            assert np.array_equal(a[r, :n].view(np.uint32), b[r, :n].view(np.uint32)), (prob.name, r)
        la = l_na.cpu().numpy()
        assert np.array_equal(la, l_ws.cpu().numpy()), prob.name
        res = dict(scores=a, lists=la, scores_only=a, lists_topk=la, code=0, detail=0)
        check_against_oracle(prob, res)


def test_noalloc_random_sequence():
    """Six seeded random problems through the static scratch back to back (each call
    finds the previous call's contents there): 1-3 requests of 1-8 rows over 1-200,000
    keys, every cache kind, k from 1 to 2048; each against idx_score_topk and the oracle."""
    for case in range(6):
        rng = np.random.default_rng(86420 + case)
        nreq = int(rng.integers(1, 4))
        contexts = [int(rng.integers(1, 200001)) for _ in range(nreq)]
        rows = [int(rng.integers(1, 9)) for _ in range(nreq)]
        k = int(rng.choice([1, 64, 300, 1024, 2048]))
        keys = str(rng.choice(["normal", "ties", "zeros", "recent"]))
        prob = make_problem(contexts, rows, seed=40000 + case, k=k, keys=keys, chain=bool(rng.random() < 0.6),
                            name=f"noalloc_random{case}")
        print(f"case {prob.name} contexts={contexts} rows={rows} k={k} keys={keys}", flush=True)
        dp = device_problem(prob)
        ld = max(1, dp.max_keys)
        s_na = torch.full((prob.rows, ld), float("nan"), dtype=torch.float32, device="cuda")
        l_na = torch.full((prob.rows, prob.k), -7, dtype=torch.int32, device="cuda")
        idx.score_topk_noalloc(dp, prob.k, s_na, l_na)
        torch.cuda.synchronize()
        ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
        s_ws, l_ws = idx.score_topk(dp, prob.k, ws)
        assert idx.device_status(ws)[0] == 0
        a, b = s_na.cpu().numpy(), s_ws.cpu().numpy()
        for r in range(prob.rows):
            n = int(prob.n_keys[r])
            assert np.array_equal(a[r, :n].view(np.uint32), b[r, :n].view(np.uint32)), (prob.name, r)
        la = l_na.cpu().numpy()
        assert np.array_equal(la, l_ws.cpu().numpy()), prob.name
        check_against_oracle(prob, dict(scores=a, lists=la, scores_only=a, lists_topk=la, code=0, detail=0))


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    """64 rows of 131,072 keys need 16 MiB + 256 B of candidate blocks: refused on the host
    with IDX_ESCRATCH before any launch (the inputs are zeros; nothing reads them)."""
    rows, pages = 64, 2048
    dev = "cuda"
    dp = idx.DeviceProblem(q=torch.zeros((rows, 64, 128), dtype=torch.int16, device=dev),
                           w=torch.zeros((rows, 64), dtype=torch.int16, device=dev),
                           k_cache=torch.zeros((pages, 64, 128), dtype=torch.uint8, device=dev),
                           k_scale=torch.zeros((pages, 64), dtype=torch.float32, device=dev),
                           page_table=torch.zeros((rows, pages), dtype=torch.int32, device=dev),
                           n_keys=torch.zeros((rows,), dtype=torch.int32, device=dev),
                           req_indptr=list(range(0, rows + 1, 4)), max_keys=pages * 64)
    s = torch.empty((rows, pages * 64), dtype=torch.float32, device=dev)
    l = torch.empty((rows, 2048), dtype=torch.int32, device=dev)
    with pytest.raises(idx.IdxError) as e:
        idx.score_topk_noalloc(dp, 2048, s, l)
    assert e.value.code == _lib.IDX_ESCRATCH
