"""Shared helpers of the GPU tests: upload a workloads.Problem, run the three entry points,
and compare with the CPU oracle."""
import numpy as np
import torch

import key_scoring_exact_amd as idx
from key_scoring_exact_amd import build as B
from oracle import check as C
from oracle import indexer as O


def device_problem(prob, req_max_keys=None, max_keys=None):
    B.ensure_built()
    return idx.DeviceProblem.from_arrays(prob.q, prob.w, prob.k_cache, prob.k_scale, prob.page_table,
                                         prob.n_keys, prob.req_indptr,
                                         max_keys=prob.max_keys if max_keys is None else max_keys,
                                         req_max_keys=req_max_keys)


def run_all(prob, ws=None, req_max_keys=None, max_keys=None):
    """Fused call, score-only call and top-k over the fused call's scores."""
    dp = device_problem(prob, req_max_keys, max_keys)
    if ws is None:
        ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    ld = max(1, dp.max_keys)
    s_f = torch.full((prob.rows, ld), float("nan"), dtype=torch.float32, device="cuda")
    l_f = torch.full((prob.rows, prob.k), -7, dtype=torch.int32, device="cuda")
    idx.score_topk(dp, prob.k, ws, scores=s_f, out=l_f)
    s_s = torch.full((prob.rows, ld), float("nan"), dtype=torch.float32, device="cuda")
    idx.score(dp, ws, scores=s_s)
    l_t = idx.topk(s_f, dp.n_keys, prob.k, dp.max_keys, ws)
    code, detail = idx.device_status(ws)
    return dict(scores=s_f.cpu().numpy(), lists=l_f.cpu().numpy(), scores_only=s_s.cpu().numpy(),
                lists_topk=l_t.cpu().numpy(), code=code, detail=detail, ws=ws)


def check_against_oracle(prob, res, ref=None, controls=False):
    """Every row: score bound vs f64, list exact vs selection of the GPU's own scores;
    score-only equals fused bitwise; top-k over given scores equals the fused list."""
    assert res["code"] == 0, f"device error {res['detail']:#x}"
    if ref is None:
        ref = O.scores(prob)
    worst = 0.0
    for r in range(prob.rows):
        n = int(prob.n_keys[r])
        g = res["scores"][r, :n]
        rep = C.check_row(r, g, res["lists"][r], ref[r], n, prob.k)
        assert rep.score_ok, (prob.name, r, n, rep.err_over_max)
        assert rep.list_ok, (prob.name, r, n, first_diff(res["lists"][r], O.select(g.astype(np.float64), n, prob.k)))
        assert np.array_equal(res["scores_only"][r, :n].view(np.uint32), g.view(np.uint32)), (prob.name, r)
        assert np.array_equal(res["lists_topk"][r], res["lists"][r]), (prob.name, r)
        if controls:
            assert all(C.negative_controls_fail(g, res["lists"][r], ref[r], n, prob.k))
        worst = max(worst, rep.err_over_max)
    return worst


def first_diff(a, b):
    d = np.nonzero(np.asarray(a) != np.asarray(b))[0]
    if len(d) == 0:
        return None
    i = int(d[0])
    return dict(index=i, got=int(a[i]), want=int(b[i]), ndiff=len(d))
