"""Device-side error paths, forced from the host so that every kernel still exits
normally: out-of-range page ids and key counts are clamped and reported, and an
uninitialised workspace is refused."""
import numpy as np
import pytest
import torch

import key_scoring_exact_amd as idx
from key_scoring_exact_amd import _lib
from workloads import make_problem

from .gpu_helpers import device_problem

pytestmark = pytest.mark.gpu


def test_bad_page_id_reported():
    prob = make_problem([5000], [2], seed=21)
    prob.page_table[1, 3] = prob.num_pages + 5       # row 1 is the longest: its table is walked
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    idx.score_topk(dp, prob.k, ws)
    code, detail = idx.device_status(ws)
    assert code == _lib.IDX_EDEVICE and detail & _lib.IDX_DERR_PAGE
    assert idx.device_status(ws) == (0, 0)           # read-and-clear


def test_bad_key_count_reported():
    prob = make_problem([3000], [1], seed=22)
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    dp.n_keys.fill_(dp.max_keys + 100)
    idx.score_topk(dp, prob.k, ws)
    code, detail = idx.device_status(ws)
    assert code == _lib.IDX_EDEVICE and detail & _lib.IDX_DERR_NKEYS
    dp.n_keys.fill_(-3)
    _, lists = idx.score_topk(dp, prob.k, ws)
    code, detail = idx.device_status(ws)
    assert code == _lib.IDX_EDEVICE and detail & _lib.IDX_DERR_NKEYS
    assert np.all(lists.cpu().numpy() == -1)         # clamped to an empty row


def test_uninitialised_workspace_refused():
    prob = make_problem([3000], [1], seed=24)
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    ws.buf.zero_()
    out = torch.full((1, prob.k), 5, dtype=torch.int32, device="cuda")
    idx.score_topk(dp, prob.k, ws, out=out)
    code, detail = idx.device_status(ws)
    assert code == _lib.IDX_EDEVICE and detail & _lib.IDX_DERR_WS
    assert np.all(out.cpu().numpy() == 5)            # nothing was written
