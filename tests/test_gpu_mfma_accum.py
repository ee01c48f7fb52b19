"""How gfx950's matrix instructions accumulate, on inputs whose products are all exact.

The scoring contraction is q[h, :] · k8[p, :] over D = 128 with bf16 q and E4M3 keys.
The indexer page computes it on MFMA chains with f32 results (Modifications item 2).
On FP8 MFMA the bf16 query would have to be split exactly into two E4M3 terms, and
the accumulation error of the FP8 instructions decides whether that path can hold
the score bound of 1e-4 of the row's largest score.  These tests measure it:

* ``test_instruction_accumulation``: C = A·Bᵀ over E4M3 codes (and their exact bf16
  images) for each instruction, error over sum |a·b| against the exact f64 sums;
* ``test_scoring_through_each_instruction``: a 4-row, 3,000-key problem scored
  through each instruction with the query split into two E4M3 terms (FP8) or kept in
  bf16, error over the row's largest oracle score.

* ``test_instruction_rate``: the dense issue rate of each instruction on this card,
  operands in registers, against the published peaks (2.5 PFLOP/s bf16, 5.0 fp8).

Run with ``-s`` to print the tables.  The bf16 instruction is held to the recursive
summation bound (terms · 2^-24 of sum |a·b|).
"""
import numpy as np
import pytest
import torch

from oracle import indexer as O
from workloads import make_problem

pytestmark = pytest.mark.gpu

MODES = {0: "v_mfma_f32_32x32x16_fp8_fp8", 1: "v_mfma_f32_32x32x64_f8f6f4", 2: "v_mfma_f32_32x32x16_bf16"}
E4M3_MAX = 448.0


def _lib():
    from tests import probes
    return probes.load()


def _run(lib, mode, a, b):
    """C = A·Bᵀ on the GPU; a [m, k], b [n, k] as uint8 codes (modes 0, 1) or uint16 bf16."""
    m, k = a.shape
    n = b.shape[0]
    dt = torch.uint8 if mode < 2 else torch.int16
    da = torch.from_numpy(np.ascontiguousarray(a).view(np.uint8 if mode < 2 else np.int16)).to("cuda")
    db = torch.from_numpy(np.ascontiguousarray(b).view(np.uint8 if mode < 2 else np.int16)).to("cuda")
    assert da.dtype == dt and db.dtype == dt
    c = torch.empty((m, n), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    rc = lib.mfma_probe(mode, da.data_ptr(), db.data_ptr(), c.data_ptr(), m, n, k, s.cuda_stream)
    assert rc == 0, f"mfma_probe returned {rc}"
    torch.cuda.synchronize()
    return c.cpu().numpy().astype(np.float64)


def _bf16_of_e4m3(codes):
    """Exact bf16 bit patterns of E4M3 codes (every finite E4M3 value is a bf16 value)."""
    v = O.decode_e4m3fn(codes).astype(np.float32)
    bits = v.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    return (bits >> 16).astype(np.uint16)


def _e4m3(x):
    """Round f32 values (|x| <= 448) to E4M3FN codes, nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.all(np.abs(x) <= E4M3_MAX)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _codes(rng, shape, kind):
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    if kind == "all finite codes":
        return rng.choice(finite, size=shape)
    g = rng.standard_normal(shape).astype(np.float32)
    if kind == "positive normal":
        g = np.abs(g)
    amax = np.abs(g).max(axis=-1, keepdims=True)
    return _e4m3(g * np.float32(E4M3_MAX) / amax * np.float32(0.999))


def _stats(err, denom):
    live = denom > 0
    rel = err[live] / denom[live]
    return float(rel.max()), float(np.median(rel))


@pytest.mark.parametrize("k", [128, 1024])
def test_instruction_accumulation(k):
    lib = _lib()
    rng = np.random.default_rng(11 + k)
    m = n = 256
    print(f"\nC = A·Bᵀ, {m} x {n} outputs, {k} terms each; error / sum|a·b| against exact f64 sums")
    print(f"{'instruction':34s} {'inputs':18s} {'max':>10s} {'median':>10s}")
    worst = {}
    for kind in ("normal", "positive normal", "all finite codes"):
        a = _codes(rng, (m, k), kind)
        b = _codes(rng, (n, k), kind)
        fa, fb = O.decode_e4m3fn(a), O.decode_e4m3fn(b)
        exact = fa @ fb.T                     # every partial sum is exact in f64
        absum = np.abs(fa) @ np.abs(fb).T
        for mode in (0, 1, 2):
            if mode < 2:
                c = _run(lib, mode, a, b)
            else:
                c = _run(lib, mode, _bf16_of_e4m3(a), _bf16_of_e4m3(b))
            mx, med = _stats(np.abs(c - exact), absum)
            worst[mode] = max(worst.get(mode, 0.0), mx)
            print(f"{MODES[mode]:34s} {kind:18s} {mx:10.3e} {med:10.3e}")
            # every instruction must compute this product (layout check): the FP8 ones
            # included, whatever their accumulation error
            assert mx < 1e-2, (MODES[mode], kind, mx)
    assert worst[2] <= k * 2.0 ** -24, worst[2]


def _split_query(q):
    """q (f64 values of bf16) -> (hi codes, lo codes, s1, s2) per row of q with
    q ≈ (hi + lo / s2) / s1: powers of two s1, s2 put each term's largest magnitude
    in [224, 448]."""
    amax = np.abs(q).max(axis=-1, keepdims=True)
    s1 = np.where(amax > 0, 2.0 ** np.floor(np.log2(E4M3_MAX / np.where(amax > 0, amax, 1.0))), 1.0)
    x = (q * s1).astype(np.float32)
    hi = _e4m3(x)
    r = x.astype(np.float64) - O.decode_e4m3fn(hi)
    ramax = np.abs(r).max(axis=-1, keepdims=True)
    s2 = np.where(ramax > 0, 2.0 ** np.floor(np.log2(E4M3_MAX / np.where(ramax > 0, ramax, 1.0))), 1.0)
    lo = _e4m3((r * s2).astype(np.float32))
    return hi, lo, s1, s2


def _combine(dots, S, W):
    """Scores from f64 dot products [H, n]: sum_h w_h · ReLU(s_p · dot)."""
    return np.einsum("h,hn->n", W, np.maximum(S[None, :] * dots, 0.0), optimize=False)


def test_scoring_through_each_instruction():
    lib = _lib()
    prob = make_problem([3000], [4], seed=7)
    dim = prob.k_cache.shape[2]
    flat = prob.k_cache.reshape(-1, dim)
    print("\nScores of 4 rows x 2,997..3,000 keys (H = 64, D = 128): max |score - oracle| / M_r")
    rows = {}
    for r in range(prob.rows):
        nk = int(prob.n_keys[r])
        slots = O.row_slots(prob.page_table[r], nk, prob.k_cache.shape[1])
        npad = (nk + 31) // 32 * 32
        kc = np.zeros((npad, dim), dtype=np.uint8)
        kc[:nk] = flat[slots]
        S = prob.k_scale.reshape(-1)[slots].astype(np.float64)
        Q = O.decode_bf16(prob.q[r])
        W = O.decode_bf16(prob.w[r])
        ref = O.row_scores(prob.q[r], prob.w[r], prob.k_cache, prob.k_scale, prob.page_table[r], nk)
        M = np.abs(ref).max()
        K8 = O.decode_e4m3fn(kc[:nk])
        hi, lo, s1, s2 = _split_query(Q)
        out = {}
        # the two-term split itself, with exact accumulation
        split = (O.decode_e4m3fn(hi) + O.decode_e4m3fn(lo) / s2) / s1
        out["split q, exact sums"] = _combine(split @ K8.T, S, W)
        out["one-term E4M3 q, exact sums"] = _combine((O.decode_e4m3fn(hi) / s1) @ K8.T, S, W)
        for mode in (0, 1):
            ch = _run(lib, mode, hi, kc)[:, :nk]
            cl = _run(lib, mode, lo, kc)[:, :nk]
            out[f"split q on {MODES[mode]}"] = _combine((ch + cl / s2) / s1, S, W)
        qb = prob.q[r].astype(np.uint16)
        c2 = _run(lib, 2, qb, _bf16_of_e4m3(kc))[:, :nk]
        out[f"bf16 q on {MODES[2]}"] = _combine(c2, S, W)
        for name, v in out.items():
            rows.setdefault(name, []).append(float(np.abs(v - ref).max() / M))
    for name, errs in rows.items():
        print(f"  {name:48s} max {max(errs):10.3e}   rows " + " ".join(f"{e:.2e}" for e in errs))
    assert max(rows["split q, exact sums"]) < 1e-6
    assert max(rows[f"bf16 q on {MODES[2]}"]) < 1e-6


def test_instruction_rate():
    from tests import probes
    lib = probes.load("mfma_rate")
    rng = np.random.default_rng(5)
    inp = torch.from_numpy(rng.integers(0, 2 ** 32, 256, dtype=np.uint64).astype(np.uint32).view(np.int32)).to("cuda")
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    import ctypes
    peak = {0: 5000.0, 1: 5000.0, 2: 2500.0, 3: 2500.0}
    names = {**MODES, 3: "v_mfma_f32_16x16x32_bf16"}
    print("\nDense issue rate, 2048 x 256 threads, two independent chains a wave")
    for mode in (2, 3, 0, 1):
        t = ctypes.c_double()
        rc = lib.mfma_rate(mode, inp.data_ptr(), out.data_ptr(), 4000, ctypes.byref(t))
        assert rc == 0, f"mfma_rate returned {rc}"
        assert torch.isfinite(out).all()
        print(f"  {names[mode]:34s} {t.value:8.1f} TFLOP/s   {t.value / peak[mode]:.3f} of the published peak")
        assert 0.2 * peak[mode] < t.value < 1.1 * peak[mode], (names[mode], t.value)
