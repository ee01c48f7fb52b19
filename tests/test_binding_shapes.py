"""The Python binding refuses tensors whose shapes disagree before any pointer reaches the
library (the kernels index by rows, heads, dim, pages and k, so a short tensor would be
read or written past its end).  CPU tensors: the shape checks run first, so these tests
need no GPU and launch nothing."""
import numpy as np
import pytest
import torch

import key_scoring_exact_amd as idx


def problem(rows=4, pages=8, max_pages=4, **over):
    kw = dict(q=torch.zeros((rows, 64, 128), dtype=torch.int16), w=torch.zeros((rows, 64), dtype=torch.int16),
              k_cache=torch.zeros((pages, 64, 128), dtype=torch.uint8),
              k_scale=torch.zeros((pages, 64), dtype=torch.float32),
              page_table=torch.zeros((rows, max_pages), dtype=torch.int32),
              n_keys=torch.zeros((rows,), dtype=torch.int32), req_indptr=[0, rows], max_keys=max_pages * 64)
    kw.update(over)
    return idx.DeviceProblem(**kw)


@pytest.mark.parametrize("field,value,match", [
    ("w", torch.zeros((3, 64), dtype=torch.int16), "w"),
    ("w", torch.zeros((4, 32), dtype=torch.int16), "w"),
    ("k_cache", torch.zeros((8, 64, 64), dtype=torch.uint8), "k_cache"),
    ("k_scale", torch.zeros((7, 64), dtype=torch.float32), "k_scale"),
    ("page_table", torch.zeros((3, 4), dtype=torch.int32), "page_table"),
    ("n_keys", torch.zeros((5,), dtype=torch.int32), "n_keys"),
    ("req_indptr", [0, 3], "req_indptr"),
    ("req_indptr", [0, 2, 2, 4], "req_indptr"),
    ("req_max_keys", [10, 20], "req_max_keys"),
    ("max_keys", 4 * 64 + 1, "max_keys"),
])
def test_problem_shapes(field, value, match):
    with pytest.raises(ValueError, match=match):
        problem(**{field: value}).struct()


def test_output_shapes():
    p = problem()
    ws = object()                       # never reached: the shape checks fail first
    with pytest.raises(ValueError, match="scores"):
        idx.score(p, ws, scores=torch.zeros((3, 256)))
    with pytest.raises(ValueError, match="out"):
        idx.score_topk(p, 16, ws, scores=torch.zeros((4, 256)), out=torch.zeros((4, 15), dtype=torch.int32))
    with pytest.raises(ValueError, match="out"):
        idx.score_topk(p, 16, ws, scores=torch.zeros((4, 256)), out=torch.zeros((3, 16), dtype=torch.int32))
    with pytest.raises(ValueError, match="slots"):
        idx.score_topk_slots(p, 16, ws, scores=torch.zeros((4, 256)), out=torch.zeros((4, 16), dtype=torch.int32),
                             slots=torch.zeros((4, 8), dtype=torch.int32))
    with pytest.raises(ValueError, match="tagged"):
        idx.score_topk_tagged(p, 16, ws, 3, scores=torch.zeros((4, 256)), out=torch.zeros((4, 16), dtype=torch.int32),
                              tagged=torch.zeros((4, 17), dtype=torch.int64))
    with pytest.raises(ValueError, match="tag"):
        idx.score_topk_tagged(p, 16, ws, 1 << 32, scores=torch.zeros((4, 256)),
                              out=torch.zeros((4, 16), dtype=torch.int32), tagged=torch.zeros((4, 16), dtype=torch.int64))
    with pytest.raises(ValueError, match="out"):
        idx.score_topk_noalloc(p, 16, torch.zeros((4, 256)), torch.zeros((4, 8), dtype=torch.int32))


def test_append_shapes():
    p = problem()
    ok = dict(new_codes=torch.zeros((4, 128), dtype=torch.uint8), new_scales=torch.zeros((4,)),
              new_pos=torch.zeros((4,), dtype=torch.int32))
    for name, bad in [("new_codes", torch.zeros((3, 128), dtype=torch.uint8)),
                      ("new_codes", torch.zeros((4, 64), dtype=torch.uint8)),
                      ("new_scales", torch.zeros((5,))), ("new_pos", torch.zeros((4, 1), dtype=torch.int32))]:
        kw = dict(ok, **{name: bad})
        with pytest.raises(ValueError, match=name):
            idx.score_topk_append(p, 16, object(), kw["new_codes"], kw["new_scales"], kw["new_pos"],
                                  scores=torch.zeros((4, 256)), out=torch.zeros((4, 16), dtype=torch.int32))


def test_topk_and_prep_shapes():
    with pytest.raises(ValueError, match="n_keys"):
        idx.topk(torch.zeros((4, 100)), torch.zeros((3,), dtype=torch.int32), 8, 100, object())
    with pytest.raises(ValueError, match="out"):
        idx.topk(torch.zeros((4, 100)), torch.zeros((4,), dtype=torch.int32), 8, 100, object(),
                 out=torch.zeros((4, 7), dtype=torch.int32))
    with pytest.raises(ValueError, match="scores"):
        idx.topk(torch.zeros((400,)), torch.zeros((4,), dtype=torch.int32), 8, 100, object())
    q = torch.zeros((2, 64, 128), dtype=torch.int16)
    with pytest.raises(ValueError, match="cos"):
        idx.prep_query(q, torch.zeros((2, 16)), torch.zeros((2, 32)), 64)
    with pytest.raises(ValueError, match="sin"):
        idx.prep_query(q, torch.zeros((2, 32)), torch.zeros((1, 32)), 64)
    with pytest.raises(ValueError):
        idx.prep_query(torch.zeros((2, 64, 64), dtype=torch.int16), None, None, 0)


def test_consistent_problem_reaches_the_device_check():
    """A problem whose shapes agree passes the shape checks and is refused only because
    its tensors are not on the device (no GPU here)."""
    with pytest.raises(ValueError, match="device"):
        problem().struct()
