"""GPU parity of index-query preparation (idx_prep_query) against the f64 oracle
(oracle/prep.py), and of preparation followed by scoring and selection.

Bound per element: |gpu - exact| <= one bf16 unit in the last place of the exact value
plus 2^-19 * (L1 norm of the head after RoPE) / sqrt(128).  The kernel rounds an f32
value once to bf16 (at most half a unit) and its f32 RoPE and 7 butterfly stages
deviate from the exact value by at most about 8 * 2^-24 of that L1 norm / sqrt(128);
the bound doubles both.  Elements whose bf16 differs from the nearest bf16 of the exact
value must stay rare (exact value within the f32 error of a rounding boundary)."""
import numpy as np
import pytest
import torch

import key_scoring_exact_amd as idx
from key_scoring_exact_amd import build as B
from oracle import prep as P
from oracle import indexer as O
from workloads import make_problem, rope_table

from .gpu_helpers import check_against_oracle, run_all

pytestmark = pytest.mark.gpu


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def run_prep(q_bits, cos, sin, rope_dim, interleaved):
    B.ensure_built()
    qd = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).cuda()
    cd = torch.from_numpy(np.ascontiguousarray(cos)).cuda() if rope_dim else None
    sd = torch.from_numpy(np.ascontiguousarray(sin)).cuda() if rope_dim else None
    out = idx.prep_query(qd, cd, sd, rope_dim, interleaved)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


def check_prep(q_bits, cos, sin, rope_dim, interleaved):
    got = O.decode_bf16(run_prep(q_bits, cos, sin, rope_dim, interleaved))
    exact = P.prep_query(q_bits, cos, sin, rope_dim, interleaved)
    x = P.rope(O.decode_bf16(q_bits), cos, sin, rope_dim, interleaved)
    l1 = np.abs(x).sum(-1, keepdims=True) / np.sqrt(128.0)
    tol = P.bf16_ulp(exact) + 2.0 ** -19 * l1
    err = np.abs(got - exact)
    assert np.all(err <= tol), (rope_dim, interleaved, float((err / tol).max()))
    nearest = torch.from_numpy(exact).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    frac = float(np.mean(got != nearest))
    assert frac < 1e-3, frac
    return frac


@pytest.mark.parametrize("rows", [1, 4, 17])
@pytest.mark.parametrize("rope_dim,interleaved", [(0, False), (2, False), (64, False), (64, True), (128, False),
                                                  (128, True), (6, True)])
def test_prep_parity(rows, rope_dim, interleaved):
    rng = np.random.default_rng(100 + rows + rope_dim + int(interleaved))
    x = rng.standard_normal((rows, 64, 128)).astype(np.float32)
    x[rows // 2] *= np.float32(300.0)                   # wide-range rows
    x[-1, :8] *= np.float32(1e-3)
    q = bf16_bits(x)
    pos = rng.integers(0, 131072, rows)
    cos, sin = rope_table(pos, rope_dim)
    print(f"case rows={rows} rope_dim={rope_dim} interleaved={interleaved}", flush=True)
    check_prep(q, cos, sin, rope_dim, interleaved)


def test_prep_special_inputs():
    # zeros stay zero; a unit vector becomes a Hadamard column; identity rotation
    q = np.zeros((2, 64, 128), dtype=np.float32)
    q[1, :, 0] = 1.0
    cos, sin = np.ones((2, 32), np.float32), np.zeros((2, 32), np.float32)
    got = O.decode_bf16(run_prep(bf16_bits(q), cos, sin, 64, False))
    assert np.all(got[0] == 0.0)
    assert np.all(np.abs(got[1]) == np.float64(torch.tensor(1 / np.sqrt(128)).to(torch.bfloat16).item()))


def test_prep_then_score_topk():
    """Preparation, then the fused call on the prepared query, against the oracle's
    prepared query (rounded to bf16) and its f64 scores."""
    prob = make_problem([40000], [4], seed=4242, name="prep40k")
    rng = np.random.default_rng(7)
    q_pre = bf16_bits(rng.standard_normal((prob.rows, 64, 128)).astype(np.float32))
    cos, sin = rope_table(np.full(prob.rows, 39999) + np.arange(prob.rows), 64)
    q_gpu = run_prep(q_pre, cos, sin, 64, False)
    exact = P.prep_query(q_pre, cos, sin, 64, False)
    q_ref = torch.from_numpy(exact).to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    prob.q = q_gpu
    res = run_all(prob)
    ref_prob = make_problem([40000], [4], seed=4242, name="prep40k")
    ref_prob.q = q_ref
    check_against_oracle(prob, res, ref=O.scores(ref_prob))
