"""hipGraph capture of the fused call: a graph of several idx_score_topk calls (over two
problems sharing one workspace) is replayed several times, with eager calls and
synchronisations between the replays, and every replay is checked bitwise against the
eager results of the same calls.  The call path records no memset node: the scoring
launch writes every candidate word the selection launch reads."""
import ctypes

import numpy as np
import pytest
import torch

import key_scoring_exact_amd as idx
from workloads import make_problem

from .gpu_helpers import device_problem

pytestmark = pytest.mark.gpu


def _call(L, st, k, ws, scores, lists, stream):
    s, _ = st
    return L.idx_score_topk(ctypes.byref(s), k, ctypes.c_void_p(scores.data_ptr()), scores.shape[1],
                            ctypes.c_void_p(lists.data_ptr()), ctypes.c_void_p(ws.ptr), ws.nbytes,
                            ctypes.c_void_p(stream.cuda_stream))


def test_graph_replays_match_eager():
    probs = [make_problem([40000], [4], seed=71), make_problem([9000, 30000], [2, 2], seed=72)]
    dps = [device_problem(p) for p in probs]
    k = probs[0].k
    rows = max(p.rows for p in probs)
    maxk = max(dp.max_keys for dp in dps)
    ws = idx.Workspace(rows, maxk, k)
    L = idx.lib()
    structs = [dp.struct() for dp in dps]
    outs = [(torch.zeros((p.rows, maxk), dtype=torch.float32, device="cuda"),
             torch.zeros((p.rows, k), dtype=torch.int32, device="cuda")) for p in probs]
    order = [0, 1, 0]

    # eager reference
    cur = torch.cuda.current_stream()
    for i in order:
        assert _call(L, structs[i], k, ws, outs[i][0], outs[i][1], cur) == 0
    torch.cuda.synchronize()
    ref = [(o[0].cpu().numpy().copy(), o[1].cpu().numpy().copy()) for o in outs]

    cs = torch.cuda.Stream()
    cs.wait_stream(cur)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for i in order:
            assert _call(L, structs[i], k, ws, outs[i][0], outs[i][1], cs) == 0
    torch.cuda.synchronize()

    for rep in range(4):
        for o in outs:                      # poison the outputs between replays
            o[0].fill_(float("nan"))
            o[1].fill_(-9)
        # eager work on the same workspace between replays
        assert _call(L, structs[1], k, ws, outs[1][0], outs[1][1], cur) == 0
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            s = o[0].cpu().numpy()
            for r in range(probs[i].rows):      # scores past n_keys[r] are not written
                n = int(probs[i].n_keys[r])
                assert np.array_equal(s[r, :n].view(np.uint32), ref[i][0][r, :n].view(np.uint32)), (rep, i, r)
            assert np.array_equal(o[1].cpu().numpy(), ref[i][1]), (rep, i)
    assert idx.device_status(ws) == (0, 0)
