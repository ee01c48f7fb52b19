"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Scores: |gpu - f64 oracle| <= 1e-4 * max_p |oracle| per row.  Lists: bit-exact against
the exact selection (score desc, position asc, emitted ascending) of the GPU's own
scores.  Every case also checks that the score-only entry point writes the same bits
and that the top-k entry point over those scores returns the same lists.
"""
import numpy as np
import pytest
import torch

from oracle import indexer as O
from workloads import make_config, make_problem
from workloads.synth import quantize_keys

from .gpu_helpers import check_against_oracle, device_problem, run_all

pytestmark = pytest.mark.gpu

SMALL_N = [0, 1, 63, 64, 65, 1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097]


@pytest.mark.parametrize("n", SMALL_N)
@pytest.mark.parametrize("k", [1, 64, 2048])
def test_small_single_row(n, k):
    prob = make_problem([n], [1], seed=1000 + n, k=k, name=f"n{n}k{k}")
    print(f"case n={n} k={k}", flush=True)
    check_against_oracle(prob, run_all(prob))


@pytest.mark.parametrize("rows", [2, 3, 4])
@pytest.mark.parametrize("n", [1, 65, 2049, 4097, 9000])
def test_small_chain(rows, n):
    prob = make_problem([n], [rows], seed=2000 + 7 * n + rows, name=f"chain{rows}x{n}")
    print(f"case rows={rows} n={n}", flush=True)
    check_against_oracle(prob, run_all(prob))


@pytest.mark.parametrize("n,k", [(24576, 2048), (24577, 2048), (40000, 2048), (40000, 64), (40000, 1),
                                 (65537, 2048), (100000, 512)])
def test_candidate_path(n, k):
    prob = make_problem([n], [4], seed=3000 + n + k, k=k, name=f"cand{n}k{k}")
    print(f"case n={n} k={k}", flush=True)
    check_against_oracle(prob, run_all(prob))


@pytest.mark.parametrize("n,rows,keys", [(262144, 4, "normal"), (524287, 1, "normal"), (524288, 4, "normal"),
                                         (200000, 2, "recent"), (262144, 2, "recent"), (524287, 1, "recent"),
                                         (300001, 3, "ties")])
def test_rows_past_128k(n, rows, keys):
    """Rows of 2-4x the 128K keys (512 to 1,024 chunks): the candidate gather runs in several
    batches; with recent keys the certificate fails and the rare path re-reads the hot
    chunks from a floor taken from the chunk headers; ties finish from the headers."""
    prob = make_problem([n], [rows], seed=6000 + n + rows, keys=keys, recent=4096, name=f"long{n}x{rows}{keys}")
    print(f"case n={n} rows={rows} keys={keys}", flush=True)
    check_against_oracle(prob, run_all(prob))


def test_mixed_requests_with_bounds():
    prob = make_problem([700, 5000, 30000, 50000, 3], [4, 1, 3, 2, 1], seed=77, name="mixed5")
    bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
    check_against_oracle(prob, run_all(prob, req_max_keys=bounds))
    check_against_oracle(prob, run_all(prob))


def test_ties_zeros_and_recent_small():
    for keys in ["ties", "zeros", "recent"]:
        for n in [3000, 40000]:
            prob = make_problem([n], [4], seed=4000 + n, keys=keys, recent=min(4096, n // 4), name=f"{keys}{n}")
            print(f"case {keys} n={n}", flush=True)
            res = run_all(prob)
            check_against_oracle(prob, res)
            if keys == "zeros":
                for r in range(prob.rows):
                    assert np.all(res["scores"][r, : int(prob.n_keys[r])] == 0)
                    assert res["lists"][r].tolist() == list(range(prob.k))


@pytest.mark.parametrize("n", [30000, 40000, 60000])
def test_ties_with_small_chunks(n):
    """The ties cache (4 key vectors, position p carries vector p mod 4) on rows that use
    128- or 256-key chunks, the last one partial: the list is the first k positions
    holding the row's largest score (a closed form over the GPU's own scores)."""
    prob = make_problem([n], [4], seed=9100 + n, keys="ties", name=f"ties{n}")
    print(f"case ties n={n}", flush=True)
    res = run_all(prob)
    check_against_oracle(prob, res)
    for r in range(prob.rows):
        v = res["scores"][r]
        nr = int(prob.n_keys[r])
        best = max(v[j] for j in range(4))
        J = [j for j in range(4) if v[j] == best]
        assert res["lists"][r].tolist() == [p for p in range(nr) if p % 4 in J][: prob.k], (n, r)


@pytest.mark.parametrize("distinct", [15, 31])
def test_recent_region_of_repeated_keys(distinct):
    """The last 4,096 positions of a 131,072-key request (scaled x8, as in the recent
    cache) repeat `distinct` key vectors, position p taking the vector of p mod
    `distinct`.  The 8 chunks there overflow their caps and publish nothing, so every
    row takes all keys of those chunks (and of the next few by threshold) with the other
    chunks' published keys.  With this seed, rows 1 and 2 cut a tie at the k-th key
    among them (273 or 132 positions share it, some selected); rows 0 and 3 end with no
    tie to cut."""
    prob = make_problem([131072], [4], seed=31, keys="recent", name=f"recent_rep{distinct}")
    n, lo = 131072, 131072 - 4096
    pt = prob.page_table[0]
    pos = np.arange(lo, n)
    src = lo + (pos - lo) % distinct
    prob.k_cache[pt[pos // 64], pos % 64] = prob.k_cache[pt[src // 64], src % 64]
    prob.k_scale[pt[pos // 64], pos % 64] = prob.k_scale[pt[src // 64], src % 64]
    print(f"case recent_rep distinct={distinct}", flush=True)
    res = run_all(prob)
    check_against_oracle(prob, res)
    g = res["scores"]
    for r in (1, 2):
        # the k-th score (GPU's own) is shared by positions in and out of the list
        s = g[r, : int(prob.n_keys[r])].astype(np.float64)
        kth = np.sort(s)[::-1][prob.k - 1]
        assert np.sum(s == kth) > 1 and np.sum(s > kth) < prob.k - 1, (distinct, r)


@pytest.mark.parametrize("recent", [2048, 12000, 40000])
def test_recent_regions_of_several_sizes(recent):
    """Recent caches whose scaled region covers 4, about 24 or about 78 chunks of a
    131,072-key request.  The chunks there publish few of the top keys, so the fast path
    fails its certificate.  The first region fits the chunks taken whole.  The larger
    ones leave hot chunks out, whose thresholds lie above the k-th key of the set taken;
    those rows re-read the chunks that may hide keys, or, when the re-read does not fit,
    select over all their scores in memory (seen on a stamped build: 12,000 takes the
    re-read in three rows and the memory select in one, 40,000 the memory select in
    three)."""
    prob = make_problem([131072], [4], seed=77 + recent, keys="recent", recent=recent,
                        name=f"recent{recent}")
    print(f"case recent={recent}", flush=True)
    res = run_all(prob)
    check_against_oracle(prob, res)


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4a", "c4b", "c4c"])
def test_full_config(name):
    prob = make_config(name)
    print(f"config {name}: rows={prob.rows} max_keys={prob.max_keys}", flush=True)
    bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
    res = run_all(prob, req_max_keys=bounds)
    ref = O.scores(prob)
    worst = check_against_oracle(prob, res, ref=ref, controls=True)
    print(f"config {name}: worst err/M = {worst:.3e}", flush=True)
    if name == "c4a":
        for r in range(prob.rows):
            v = res["scores"][r]
            n = int(prob.n_keys[r])
            best = max(v[j] for j in range(4))
            J = [j for j in range(4) if v[j] == best]
            assert res["lists"][r].tolist() == [p for p in range(n) if p % 4 in J][: prob.k]
    if name == "c4b":
        assert all(res["lists"][r].tolist() == list(range(2048)) for r in range(prob.rows))


def test_deterministic_and_layout_invariant():
    prob = make_problem([50000], [4], seed=5)
    a = run_all(prob)
    b = run_all(prob, ws=a["ws"])
    assert np.array_equal(a["scores"].view(np.uint32), b["scores"].view(np.uint32))
    assert np.array_equal(a["lists"], b["lists"])
    # the same logical keys on a different physical page layout: identical scores
    perm = np.random.default_rng(1).permutation(prob.num_pages)
    kc = np.empty_like(prob.k_cache); ks = np.empty_like(prob.k_scale)
    kc[perm] = prob.k_cache; ks[perm] = prob.k_scale
    prob2 = make_problem([50000], [4], seed=5)
    prob2.k_cache, prob2.k_scale = kc, ks
    prob2.page_table = perm[prob.page_table].astype(np.int32)
    c = run_all(prob2)
    assert np.array_equal(a["scores"].view(np.uint32), c["scores"].view(np.uint32))
    assert np.array_equal(a["lists"], c["lists"])


def test_stale_workspace_contents_are_ignored():
    """A call reads back only the candidate words its own scoring launch wrote: a
    workspace whose body (past its 256-byte header) holds random bytes gives the
    same results, over the row kinds (all keys, candidates, short rows, re-read
    chunks)."""
    import key_scoring_exact_amd as idx
    ws = idx.Workspace(16, 60000, 2048)
    gen = torch.Generator(device="cuda").manual_seed(12)
    for prob in [make_problem([60000], [4], seed=9), make_problem([700, 9000, 40000], [2, 4, 3], seed=10),
                 make_problem([40000], [4], seed=11, keys="recent", recent=4096)]:
        body = ws.buf[ws.offset + 256: ws.offset + ws.nbytes]
        body.copy_(torch.randint(0, 256, body.shape, dtype=torch.uint8, device="cuda", generator=gen))
        res = run_all(prob, ws=ws)
        check_against_oracle(prob, res)


@pytest.mark.parametrize("cut", [11072, 31072])
def test_rows_below_the_call_bound_ignore_older_blocks(cut):
    """Rows shorter than the call's key bound (no per-request bound) read only the
    candidate blocks of their own chunks: the workspace first holds the blocks of a call
    over the full rows, which look valid past the short rows (cut 11,072: 119,997..
    120,000 keys, the block size of the bound; cut 31,072: a larger block)."""
    import key_scoring_exact_amd as idx
    full = make_problem([131072], [4], seed=21, name="full")
    ws = idx.Workspace(full.rows, full.max_keys, full.k)
    check_against_oracle(full, run_all(full, ws=ws))
    short = make_problem([131072], [4], seed=21, name=f"short{cut}")
    short.n_keys = (full.n_keys - cut).astype(np.int32)
    print(f"case cut={cut} n={short.n_keys.tolist()}", flush=True)
    res = run_all(short, ws=ws, max_keys=full.max_keys)
    check_against_oracle(short, res)


@pytest.mark.parametrize("rows,n", [(5, 3000), (8, 9000), (8, 40000), (6, 131072)])
def test_long_verify_chains(rows, n):
    """More than four verify rows in a request: the rows are scored in groups of at most
    four over the request's pages (each group walks the pages once)."""
    prob = make_problem([n], [rows], seed=8000 + n + rows, name=f"chain{rows}x{n}")
    print(f"case rows={rows} n={n}", flush=True)
    check_against_oracle(prob, run_all(prob))


def test_mixed_requests_with_long_chains():
    prob = make_problem([9000, 1500, 30000], [8, 1, 5], seed=88, name="mixed_long")
    bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
    check_against_oracle(prob, run_all(prob, req_max_keys=bounds))


@pytest.mark.parametrize("contexts,rows", [([3000], [4]), ([131072], [4]), ([1500, 40000, 9000], [2, 3, 8])])
def test_slot_output(contexts, rows):
    """idx_score_topk_slots: the same scores and lists as idx_score_topk, and each list
    entry as its physical cache slot through the row's own page-table row."""
    import key_scoring_exact_amd as idx
    from .gpu_helpers import device_problem
    prob = make_problem(contexts, rows, seed=9100 + sum(contexts), name=f"slots{contexts}")
    print(f"case slots {contexts} {rows}", flush=True)
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    sc, ls, sl = idx.score_topk_slots(dp, prob.k, ws)
    sc2, ls2 = idx.score_topk(dp, prob.k, ws)
    assert idx.device_status(ws)[0] == 0
    ls, sl = ls.cpu().numpy(), sl.cpu().numpy()
    assert np.array_equal(ls, ls2.cpu().numpy())
    a, b = sc.cpu().numpy().view(np.uint32), sc2.cpu().numpy().view(np.uint32)
    for r in range(prob.rows):                     # positions past n_keys are not written
        n = int(prob.n_keys[r])
        assert np.array_equal(a[r, :n], b[r, :n]), r
    assert np.array_equal(sl, O.list_slots(prob, ls))
    res = dict(scores=sc.cpu().numpy(), lists=ls, scores_only=sc.cpu().numpy(), lists_topk=ls, code=0, detail=0)
    check_against_oracle(prob, res)


@pytest.mark.parametrize("case", range(8))
def test_slot_output_random(case):
    """idx_score_topk_slots on seeded random problems (1-3 requests of 1-8 rows over
    1-200,000 keys, every cache kind, k from 1 to 2048, spare pool pages, chains or
    full-context rows): lists and scores as idx_score_topk, slots as the oracle's map."""
    import key_scoring_exact_amd as idx
    from .gpu_helpers import device_problem
    rng = np.random.default_rng(97531 + case)
    nreq = int(rng.integers(1, 4))
    contexts = [int(rng.integers(1, 200001)) for _ in range(nreq)]
    rows = [int(rng.integers(1, 9)) for _ in range(nreq)]
    k = int(rng.choice([1, 64, 300, 1024, 2048]))
    keys = str(rng.choice(["normal", "ties", "zeros", "recent"]))
    chain = bool(rng.random() < 0.6)
    prob = make_problem(contexts, rows, seed=60000 + case, k=k, keys=keys, chain=chain,
                        pad_pages=int(rng.integers(0, 5)), name=f"slots_random{case}")
    print(f"case slots_random{case} contexts={contexts} rows={rows} k={k} keys={keys} chain={chain}", flush=True)
    dp = device_problem(prob)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    sc, ls, sl = idx.score_topk_slots(dp, prob.k, ws)
    sc2, ls2 = idx.score_topk(dp, prob.k, ws)
    assert idx.device_status(ws)[0] == 0
    ls, sl = ls.cpu().numpy(), sl.cpu().numpy()
    assert np.array_equal(ls, ls2.cpu().numpy())
    a, b = sc.cpu().numpy().view(np.uint32), sc2.cpu().numpy().view(np.uint32)
    for r in range(prob.rows):
        n = int(prob.n_keys[r])
        assert np.array_equal(a[r, :n], b[r, :n]), r
    assert np.array_equal(sl, O.list_slots(prob, ls))
    res = dict(scores=sc.cpu().numpy(), lists=ls, scores_only=sc.cpu().numpy(), lists_topk=ls, code=0, detail=0)
    check_against_oracle(prob, res)


@pytest.mark.parametrize("case", range(24))
def test_random_sweep(case):
    """Seeded random problems: 1-4 requests of 1-8 rows, 0-60,000 keys a request, every
    key cache kind, k from 1 to 2048, chains or full-context rows, spare pool pages."""
    rng = np.random.default_rng(12345 + case)
    nreq = int(rng.integers(1, 5))
    contexts = [int(rng.choice([0, 1, 63, 64, 65, 2047, 2048, 2049]) if rng.random() < 0.3
                    else rng.integers(1, 60000)) for _ in range(nreq)]
    rows = [int(rng.integers(1, 9)) for _ in range(nreq)]
    k = int(rng.choice([1, 7, 64, 300, 1024, 2048]))
    keys = str(rng.choice(["normal", "normal", "ties", "zeros", "recent"]))
    chain = bool(rng.random() < 0.7)
    prob = make_problem(contexts, rows, seed=50000 + case, k=k, keys=keys, recent=int(rng.integers(64, 8192)),
                        chain=chain, pad_pages=int(rng.integers(0, 5)), name=f"sweep{case}")
    print(f"case sweep{case} contexts={contexts} rows={rows} k={k} keys={keys} chain={chain}", flush=True)
    bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
    check_against_oracle(prob, run_all(prob, req_max_keys=bounds if case % 2 else None))


@pytest.mark.parametrize("case", range(16))
def test_random_sweep_long(case):
    """Seeded random problems on the candidate path: 1-2 requests of 1-4 rows over
    60,000-300,000 keys, every key cache kind, k from 1 to 2048 (so chunk blocks of one,
    two and four 32-slot groups), chains or full-context rows, spare pool pages."""
    rng = np.random.default_rng(24680 + case)
    nreq = int(rng.integers(1, 3))
    contexts = [int(rng.integers(60000, 300001)) for _ in range(nreq)]
    rows = [int(rng.integers(1, 5)) for _ in range(nreq)]
    k = int(rng.choice([1, 7, 64, 300, 1024, 2048]))
    keys = str(rng.choice(["normal", "normal", "ties", "zeros", "recent"]))
    chain = bool(rng.random() < 0.7)
    prob = make_problem(contexts, rows, seed=70000 + case, k=k, keys=keys, recent=int(rng.integers(64, 16384)),
                        chain=chain, pad_pages=int(rng.integers(0, 5)), name=f"sweeplong{case}")
    print(f"case sweeplong{case} contexts={contexts} rows={rows} k={k} keys={keys} chain={chain}", flush=True)
    bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
    check_against_oracle(prob, run_all(prob, req_max_keys=bounds if case % 2 else None))


@pytest.mark.parametrize("k", [2048, 512])
def test_fast_path_block_sizes(k):
    """One launch of 512-key chunks (set by the 131,072-key request) whose other requests
    hold 40,000 and 32,768 keys: at k = 2048 their chunks publish blocks of 1, 2 and 4
    slot groups, and every row still fits the fast path, so the chunk headers sit in
    lanes 0, 16, 32 and 48, in lanes 0 and 32, or in lane 0 of each wave (k = 512: one
    group everywhere, fewer candidates a chunk)."""
    prob = make_problem([131072, 40000, 32768], [1, 4, 4], seed=9600 + k, k=k, name=f"blocks{k}")
    print(f"case fast-path block sizes k={k}", flush=True)
    check_against_oracle(prob, run_all(prob))


@pytest.mark.parametrize("n,distinct", [(8192, 1000), (20000, 1500), (40000, 2500), (131072, 2000)])
def test_repeated_key_vectors(n, distinct):
    """Position p carries key vector p mod `distinct` of normal keys, so every score value
    repeats about n / distinct times, each chunk holding at most one copy.  No chunk
    overflows and no tie is massive, yet the k-th key is shared by positions in and out
    of the list (checked on the oracle's scores: 8 to 66 positions share it).  The
    selection from all scores (8,192 and 20,000 keys), the gathered candidates (40,000)
    and the candidate fast path (131,072) each cut that tie in position order."""
    prob = make_problem([n], [4], seed=9700 + n, name=f"repeat{distinct}")
    pt = prob.page_table[0]
    pos = np.arange(distinct, n)
    src = pos % distinct
    prob.k_cache[pt[pos // 64], pos % 64] = prob.k_cache[pt[src // 64], src % 64]
    prob.k_scale[pt[pos // 64], pos % 64] = prob.k_scale[pt[src // 64], src % 64]
    print(f"case repeated key vectors n={n} distinct={distinct}", flush=True)
    res = run_all(prob)
    check_against_oracle(prob, res)
    cut = 0
    for r in range(prob.rows):
        s = res["scores"][r, : int(prob.n_keys[r])].astype(np.float64)
        kth = np.sort(s)[::-1][prob.k - 1]
        cut += int(np.sum(s == kth) > 1 and np.sum(s > kth) < prob.k - 1)
    assert cut > 0, (n, distinct)


@pytest.mark.parametrize("n", [40000, 131072])
def test_ties_at_random_positions(n):
    """The ties cache with the 4 vectors laid out at seeded random positions: each block of
    512 positions draws its vectors from its own Dirichlet(0.3) mix, so a row's best
    vector is dense in some chunks and sparse (fewer copies than the chunk's candidate
    rank) in others.  The list is the first k positions holding the row's largest score
    (a closed form over the GPU's own scores), and the oracle check holds."""
    prob = make_problem([n], [4], seed=9800 + n, keys="ties", name=f"ties_rand{n}")
    rng = np.random.default_rng(9900 + n)
    pt = prob.page_table[0]
    reps = [(pt[j // 64], j % 64) for j in range(4)]             # positions 0..3 hold vectors 0..3
    vc = [prob.k_cache[a, b].copy() for a, b in reps]
    vs = [prob.k_scale[a, b] for a, b in reps]
    vec = np.empty(n, dtype=np.int64)
    for b0 in range(0, n, 512):
        mix = rng.dirichlet([0.3] * 4)
        vec[b0:b0 + 512] = rng.choice(4, size=min(512, n - b0), p=mix)
    vec[:4] = np.arange(4)
    for p in range(n):
        prob.k_cache[pt[p // 64], p % 64] = vc[vec[p]]
        prob.k_scale[pt[p // 64], p % 64] = vs[vec[p]]
    print(f"case ties at random positions n={n}", flush=True)
    res = run_all(prob)
    check_against_oracle(prob, res)
    for r in range(prob.rows):
        v = res["scores"][r]
        nr = int(prob.n_keys[r])
        best = max(v[j] for j in range(4))
        hold = [p for p in range(nr) if v[p] == best]
        assert len(hold) >= prob.k, (n, r, len(hold))
        assert res["lists"][r].tolist() == hold[: prob.k], (n, r)


def test_many_requests_to_the_group_limit():
    """256 row groups in one call, the ABI's limit: 214 one-row requests, 30 two-row
    chains, 6 five-row chains (two groups each), contexts 0 to 40,000 keys, with and
    without per-request key bounds; through idx_score_topk, idx_topk and the slot map."""
    rng = np.random.default_rng(424242)
    rows = [1] * 214 + [2] * 30 + [5] * 6
    order = rng.permutation(len(rows))
    rows = [rows[i] for i in order]
    contexts = []
    for i in range(len(rows)):
        u = rng.random()
        contexts.append(int(rng.choice([0, 1, 2047, 2048, 2049])) if u < 0.1 else
                        int(rng.integers(25000, 40001)) if u < 0.2 else int(rng.integers(1, 12000)))
    groups = sum((r + 3) // 4 for r in rows)
    assert groups == 256
    prob = make_problem(contexts, rows, seed=4243, chain=True, name="groups256")
    print(f"case 256 groups: rows={prob.rows} key_rows={prob.key_rows()}", flush=True)
    bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
    ref = O.scores(prob)
    check_against_oracle(prob, run_all(prob, req_max_keys=bounds), ref=ref)
    check_against_oracle(prob, run_all(prob), ref=ref)
    import key_scoring_exact_amd as idx
    dp = device_problem(prob, req_max_keys=bounds)
    ws = idx.Workspace(prob.rows, dp.max_keys, prob.k)
    _, ls, sl = idx.score_topk_slots(dp, prob.k, ws)
    assert idx.device_status(ws)[0] == 0
    assert np.array_equal(sl.cpu().numpy(), O.list_slots(prob, ls.cpu().numpy()))


def test_topk_over_more_than_1024_rows():
    """idx_topk over 1,100 rows of given scores runs two launches of row groups; rows of
    0 to 30,000 keys (some past the all-keys bound, which publish candidates first), with
    ties at the k-th score in some rows.  Each list is exact over its row's scores."""
    import key_scoring_exact_amd as idx
    rng = np.random.default_rng(77)
    rows, ld, k = 1100, 30000, 2048
    n = rng.integers(0, 6000, size=rows).astype(np.int32)
    long_rows = rng.choice(rows, size=40, replace=False)
    n[long_rows] = rng.integers(24577, ld + 1, size=40)
    n[:3] = [0, 2048, 2049]
    sc = rng.standard_normal((rows, ld)).astype(np.float32)
    sc[10::7, :] = np.round(sc[10::7, :] * 4) / 4            # coarse values: ties at the threshold
    s_d = torch.from_numpy(sc).cuda()
    n_d = torch.from_numpy(n).cuda()
    ws = idx.Workspace(rows, ld, k)
    print(f"case topk rows={rows} ld={ld}", flush=True)
    out = idx.topk(s_d, n_d, k, ld, ws).cpu().numpy()
    assert idx.device_status(ws)[0] == 0
    for r in range(rows):
        want = O.select(sc[r].astype(np.float64), int(n[r]), k)
        assert np.array_equal(out[r], want), (r, int(n[r]))


def _given_scores(kind, rows, ld, rng):
    if kind == "signed zeros":                  # the k-th score a zero of either sign
        x = rng.standard_normal((rows, ld)).astype(np.float32)
        z = rng.random((rows, ld)) < 0.7
        x[z] = np.where(rng.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
        return x
    if kind == "subnormals":                    # mostly subnormal magnitudes, both signs
        bits = rng.integers(1, 1 << 23, size=(rows, ld), dtype=np.int64).astype(np.uint32)
        bits |= (rng.random((rows, ld)) < 0.5).astype(np.uint32) << 31
        x = bits.view(np.float32).copy()
        x[rng.random((rows, ld)) < 0.05] = np.float32(0.0)
        return x
    if kind == "wide":                          # magnitudes over the whole f32 range
        e = rng.uniform(-44.0, 38.0, size=(rows, ld))
        return (np.sign(rng.standard_normal((rows, ld))) * 10.0 ** e).astype(np.float32)
    if kind == "three values":
        return rng.choice(np.array([-1.5, 0.25, 2.0], dtype=np.float32), size=(rows, ld))
    # near the largest finite f32
    return (np.float32(3.0e38) * rng.uniform(-1.1, 1.1, size=(rows, ld))).astype(np.float32)


@pytest.mark.parametrize("kind", ["signed zeros", "subnormals", "wide", "three values", "near max"])
def test_topk_given_scores_values(kind):
    """idx_topk over caller-given scores with values the scoring never makes: zeros of
    both signs (equal as reals, the lower position first), subnormals, magnitudes over
    the whole f32 range, three distinct values, values near the largest finite f32.
    Rows of 0, 1, 2,047-2,049, 24,576-24,577 and 100,000-200,000 keys (all-scores and
    candidate paths).  Each list equals the oracle's exact selection."""
    import key_scoring_exact_amd as idx
    rng = np.random.default_rng(4242 + len(kind))
    ld = 200000
    n = np.array([0, 1, 2047, 2048, 2049, 24576, 24577, 100000, 200000], dtype=np.int32)
    rows = len(n)
    sc = _given_scores(kind, rows, ld, rng)
    assert np.isfinite(sc).all()
    for k in (1, 300, 2048):
        print(f"case topk values={kind} k={k}", flush=True)
        ws = idx.Workspace(rows, ld, k)
        out = idx.topk(torch.from_numpy(sc).cuda(), torch.from_numpy(n).cuda(), k, ld, ws).cpu().numpy()
        assert idx.device_status(ws)[0] == 0
        for r in range(rows):
            want = O.select(sc[r].astype(np.float64), int(n[r]), k)
            assert np.array_equal(out[r], want), (kind, k, r, int(n[r]))


def _hot_ties(n, rows, k, seed, hot=4096):
    """Normal keys, except that positions n - hot .. n - 1 carry one of four key vectors
    (position p the vector p mod 4), scaled 8x: each row's top keys are four tie groups of
    hot / 4 positions in the hot chunks, whose candidate blocks overflow."""
    prob = make_problem([n], [rows], seed=seed, k=k, name=f"hotties{n}x{rows}")
    # four vectors near sum_{r,h} max(w, 0) q: a large positive score in every row
    q = O.decode_bf16(prob.q[:rows])
    w = np.maximum(O.decode_bf16(prob.w[:rows]), 0.0)
    base = np.einsum("rh,rhd->d", w, q)
    noise = np.random.default_rng(seed + 1).standard_normal((4, base.size))
    vecs = base / np.linalg.norm(base) + 0.2 * noise / np.sqrt(base.size)
    vecs *= 8.0 * np.sqrt(base.size) / np.linalg.norm(vecs, axis=1, keepdims=True)
    codes, scales = quantize_keys(vecs.astype(np.float32))
    ps = np.arange(n - hot, n)
    for r in range(rows):                 # every row of the chain reads the same pages
        pages = prob.page_table[r][ps // 64]
        prob.k_cache[pages, ps % 64] = codes[ps % 4]
        prob.k_scale[pages, ps % 64] = scales[ps % 4]
    return prob


@pytest.mark.parametrize("n", [100000, 200000, 300000])
def test_rare_path_tie_cut(n):
    """The certificate fails (the hot chunks overflow) and the k-th key falls inside a tie
    group of the hot positions: the rare path re-reads the hot chunks and keeps the lowest
    positions of the cut group, at row lengths below and above 131,072 keys."""
    prob = _hot_ties(n, 2, 2000, seed=9100 + n)
    print(f"case n={n}", flush=True)
    res = run_all(prob)
    check_against_oracle(prob, res)
    for r in range(prob.rows):
        nr = int(prob.n_keys[r])
        g = res["scores"][r, :nr]
        kth = np.sort(g)[::-1][prob.k - 1]
        assert np.count_nonzero(g == kth) > 1 and np.count_nonzero(g > kth) < prob.k    # a tie is cut
