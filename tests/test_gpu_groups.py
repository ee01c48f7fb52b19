"""Row-group shapes the configuration sweeps do not reach: groups with fewer chunks than
rows, groups whose rows have no keys, grids of many groups with more workgroups than
compute units, and back-to-back calls on one workspace and stream."""
import numpy as np
import pytest
import torch

from workloads import make_problem

from .gpu_helpers import check_against_oracle, run_all

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 40, 64, 65, 200, 2049, 3000])
def test_groups_with_fewer_chunks_than_rows(n):
    """Rows of up to a few chunks: a 4-row group of 1..47 chunks."""
    prob = make_problem([n], [4], seed=31000 + n, name=f"short{n}")
    print(f"case n={n}", flush=True)
    res = run_all(prob)
    check_against_oracle(prob, res)


def test_groups_with_empty_rows():
    """A request whose rows hold no keys between two that do: its lists are all -1."""
    prob = make_problem([5000, 0, 3000], [4, 3, 2], seed=31100, name="empty-mid")
    assert prob.n_keys[4:7].max() == 0
    res = run_all(prob)
    check_against_oracle(prob, res)
    assert np.all(res["lists"][4:7] == -1)


def test_many_groups_and_a_second_round_of_workgroups():
    """64 requests of 2 rows over 6,000 keys (chunks of 64 keys): 64 groups of 94 chunks,
    6,016 workgroups on 256 compute units, with selectors waiting in every group; then
    the same workspace for a call of another shape."""
    import key_scoring_exact_amd as idx
    ws = idx.Workspace(128, 131072, 2048)
    prob = make_problem([6000] * 64, [2] * 64, seed=31200, chain=False, name="many-groups")
    res = run_all(prob, ws=ws)
    check_against_oracle(prob, res)
    prob2 = make_problem([131072, 9000], [4, 2], seed=31201, name="after")
    res2 = run_all(prob2, ws=ws)
    check_against_oracle(prob2, res2)


def test_repeated_calls_give_the_same_lists():
    """Back-to-back calls on one workspace and stream: every call's lists are the first
    call's."""
    import key_scoring_exact_amd as idx
    prob = make_problem([40000, 7000], [4, 3], seed=31300, name="repeat")
    from .gpu_helpers import device_problem
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    first = None
    for _ in range(20):
        _, lists = idx.score_topk(dp, prob.k, ws)
        got = lists.cpu().numpy()
        if first is None:
            first = got
        assert np.array_equal(got, first)
    torch.cuda.synchronize()
    assert idx.device_status(ws)[0] == 0
