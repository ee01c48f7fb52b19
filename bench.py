"""Benchmark of the score + exact top-2048 call on one MI355X.

A step is one idx_score_topk call: every stage of the hot path (page walk and key
streaming, the bf16 MFMA contraction, the ReLU / head-weighted epilogue, the radix keys,
the per-chunk candidate publication, the threshold and the ascending emission), over the
4-row x 131,072-key verify workload: one request, rows seeing 131,069..131,072 keys, 64
heads of dimension 128, pages of 64 FP8-E4M3 keys with per-key f32 scales on a seeded
random page permutation, k = 2048.  Inputs are synthetic and resident in HBM before the
timed region.  The calls rotate over enough copies of the key cache (512 MiB, twice the
256 MiB last-level cache) that keys come from HBM.

Timing protocol.  W warm-up calls, then the K steps are timed three ways with HIP events
on the launch stream:
- back to back on the stream (host launch cost included);
- as replays of hipGraphs of exactly K captured calls: one replay is one trial of K
  steps.  Each pass runs `trials` replays of the fused call and `trials` replays of the
  scores-only call (idx_score), the two alternating in order from pass to pass.
  Consecutive replays use graphs over different cache copies, so the rotation covers
  every copy.  ms_per_step is the median over all fused trials (min and mean reported);
- the scores-only figure the same way.

One JSON line is printed.  `roofline` is for the whole call (both launches; the scoring
launch dominates), against dense bf16 MFMA, the contraction's own dtype;
`roofline_score_kernel` times the scoring launch alone through idx_score.  `extra`
carries the 8,192-key x 4-row verify workload under the same protocol.  The CPU baseline
is the oracle as it stands, run over the workload's page blocks on every host core.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
MALL_ROTATE_MIB = 512          # key-cache bytes the calls rotate over: twice the last-level cache


def algorithmic_bytes(rows_n, pages, rows, k, heads=64, dim=128):
    """Bytes the call must move at least: every key of the request once (FP8 codes
    and f32 scale), one page-table row, the queries, head weights and key counts,
    the f32 scores written and the int32 lists written."""
    keys = pages * 64
    return (keys * dim + keys * 4 + pages * 4 + rows * heads * dim * 2 + rows * heads * 2 + rows * 4
            + sum(rows_n) * 4 + rows * k * 4)


def measured_traffic(build_hash16, workload):
    """HBM bytes per call (both launches) from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, scaled by a copy kernel's readings), if it was taken on a
    library built from the current sources and on this workload; else None."""
    path = os.path.join(ROOT, "profiles", "score_select_c2_traffic.txt")
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return None
    d = {}
    for ln in lines:
        if ln.startswith("#") or ":" not in ln:
            continue
        key, val = ln.split(":", 1)
        d[key.strip()] = val.strip()
    if d.get("library_build_sha256_16") != build_hash16 or d.get("workload") != workload:
        return None
    try:
        return int(d["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Bench:
    """One workload on the device: its key-cache copies, outputs and marshalled calls."""

    def __init__(self, idx, prob, rotate_mib, max_copies):
        import ctypes
        import torch
        self.prob = prob
        bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
        base = idx.DeviceProblem.from_arrays(prob.q, prob.w, prob.k_cache, prob.k_scale, prob.page_table,
                                             prob.n_keys, prob.req_indptr, max_keys=prob.max_keys,
                                             req_max_keys=bounds)
        copy_bytes = base.k_cache.numel() + base.k_scale.numel() * 4
        self.copies = max(1, min(max_copies, math.ceil(rotate_mib * (1 << 20) / copy_bytes)))
        kcs = [base.k_cache] + [base.k_cache.clone() for _ in range(self.copies - 1)]
        kss = [base.k_scale] + [base.k_scale.clone() for _ in range(self.copies - 1)]
        self.probs = [idx.DeviceProblem(q=base.q, w=base.w, k_cache=kcs[i], k_scale=kss[i],
                                        page_table=base.page_table, n_keys=base.n_keys,
                                        req_indptr=base.req_indptr, max_keys=base.max_keys,
                                        req_max_keys=base.req_max_keys) for i in range(self.copies)]
        self.base = base
        self.ws = idx.Workspace(prob.rows, base.max_keys, prob.k)
        self.scores = torch.empty((prob.rows, base.max_keys), dtype=torch.float32, device="cuda")
        self.lists = torch.empty((prob.rows, prob.k), dtype=torch.int32, device="cuda")
        self.L = idx.lib()
        self.idx = idx
        self.structs = [p.struct() for p in self.probs]     # marshalled once; the loops only call the ABI
        self.sptr = ctypes.c_void_p(self.scores.data_ptr())
        self.lptr = ctypes.c_void_p(self.lists.data_ptr())
        self.wsp = ctypes.c_void_p(self.ws.ptr)
        self.ctypes = ctypes

    def fused(self, i, st):
        s, _ = self.structs[i % self.copies]
        rc = self.L.idx_score_topk(self.ctypes.byref(s), self.prob.k, self.sptr, self.scores.shape[1], self.lptr,
                                   self.wsp, self.ws.nbytes, self.ctypes.c_void_p(st))
        if rc:
            raise self.idx.IdxError(rc, "idx_score_topk")

    def score_only(self, i, st):
        s, _ = self.structs[i % self.copies]
        rc = self.L.idx_score(self.ctypes.byref(s), self.sptr, self.scores.shape[1], self.wsp, self.ws.nbytes,
                              self.ctypes.c_void_p(st))
        if rc:
            raise self.idx.IdxError(rc, "idx_score")


def stream_time(torch, stream, fn, calls, warmup):
    """us per call, back to back on the stream: HIP events around exactly `calls` calls."""
    for i in range(warmup):
        fn(i, stream.cuda_stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(calls):
        fn(i, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / calls


def capture(torch, stream, fn, calls, first):
    """A hipGraph of `calls` calls (call i uses key copy first + i)."""
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for i in range(calls):
            fn(first + i, cs.cuda_stream)
    torch.cuda.synchronize()
    return g


def graph_trials(torch, stream, bench, calls, trials, passes):
    """Per-call us of each trial (one replay of `calls` calls), fused and scores-only, the
    two alternating in order from pass to pass; graphs cycle over the key copies."""
    ngraph = max(1, math.ceil(bench.copies / calls))
    gf = [capture(torch, stream, bench.fused, calls, j * calls) for j in range(ngraph)]
    gs = [capture(torch, stream, bench.score_only, calls, j * calls) for j in range(ngraph)]
    for g in gf + gs:                                   # one warm replay of each
        g.replay()
    torch.cuda.synchronize()
    out = {"fused": [], "score": []}
    turn = 0
    for p in range(passes):
        order = ["fused", "score"] if p % 2 == 0 else ["score", "fused"]
        for name in order:
            graphs = gf if name == "fused" else gs
            for _ in range(trials):
                g = graphs[turn % ngraph]
                turn += 1
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                out[name].append(e0.elapsed_time(e1) * 1e3 / calls)
    del gf, gs
    return out


def summary(xs):
    return {"median": statistics.median(xs), "min": min(xs), "mean": statistics.fmean(xs), "n": len(xs)}


def cpu_oracle_baseline(prob, seconds):
    """The oracle (oracle/indexer.py, unchanged) over the whole workload on every host core:
    each row's positions in page-aligned blocks (the oracle's row_scores on the block's
    page-table suffix: per-position arithmetic unchanged, results bit for bit those of
    one call over the row), then the oracle's selection of each row, on a thread pool.
    Repeated until `seconds` have passed; returns (seconds a pass, threads, passes)."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    from oracle import indexer as O
    threads = len(os.sched_getaffinity(0))
    tasks = []
    for r in range(prob.rows):
        n = int(prob.n_keys[r])
        pages = (n + 63) // 64
        step = max(1, math.ceil(pages / (2 * threads)))
        for j in range(0, pages, step):
            tasks.append((r, j, min(pages, j + step)))

    def block(t):
        r, j0, j1 = t
        n = int(prob.n_keys[r])
        p0, p1 = j0 * 64, min(n, j1 * 64)
        return r, p0, O.row_scores(prob.q[r], prob.w[r], prob.k_cache, prob.k_scale, prob.page_table[r][j0:], p1 - p0)

    passes, t0 = 0, time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        while True:
            rows = [np.empty(int(prob.n_keys[r])) for r in range(prob.rows)]
            for r, p0, v in ex.map(block, tasks):
                rows[r][p0:p0 + len(v)] = v
            lists = list(ex.map(lambda r: O.select(rows[r], int(prob.n_keys[r]), prob.k), range(prob.rows)))
            passes += 1
            if time.perf_counter() - t0 >= seconds:
                break
    return (time.perf_counter() - t0) / passes, threads, passes, rows, np.stack(lists)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200, help="K: calls a timed trial covers")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--trials", type=int, default=7, help="graph replays per pass and entry point")
    ap.add_argument("--passes", type=int, default=2, help="alternating passes (fused first, then scores first)")
    ap.add_argument("--rotate-mib", type=int, default=MALL_ROTATE_MIB,
                    help="key-cache bytes the calls rotate over (0 = one copy, warm)")
    ap.add_argument("--config", default="c2", help="workload recipe (c2 is the benchmark)")
    ap.add_argument("--no-extra", action="store_true", help="skip the 8K-context figure")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle over the workload until this much time has passed")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, run a plain f32 copy-shaped kernel (torch.neg) over this "
                         "many MiB five times: the calibration dispatch for the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; sharding over several GPUs is "
                                   "designed but not built", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import key_scoring_exact_amd as idx
    from key_scoring_exact_amd import build as B
    from workloads import make_config

    B.ensure_built()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    L = idx.lib()
    build_hash = L.idx_build_hash().decode()

    def measure(name, calls, warmup):
        prob = make_config(name)
        bench = Bench(idx, prob, args.rotate_mib, max_copies=1 << 20)
        us_stream = stream_time(torch, stream, bench.fused, calls, warmup)
        us_stream_score = stream_time(torch, stream, bench.score_only, calls, warmup)
        tr = graph_trials(torch, stream, bench, calls, args.trials, args.passes)
        code, detail = idx.device_status(bench.ws)
        if code != 0:
            raise RuntimeError(f"device error {detail:#x}")
        return prob, bench, us_stream, us_stream_score, tr

    prob, bench, us_stream, us_stream_score, tr = measure(args.config, args.steps, args.warmup)
    fused, score = summary(tr["fused"]), summary(tr["score"])
    us_call = fused["median"]

    # index-query preparation (RoPE on 64 of 128 dims, then the Hadamard transform) of the
    # same rows, the step before the scoring launch: one launch, timed back to back
    import ctypes
    from workloads import rope_table
    cos_t, sin_t = rope_table(prob.n_keys.astype(np.int64) - 1, 64)
    cos_d, sin_d = torch.from_numpy(cos_t).cuda(), torch.from_numpy(sin_t).cuda()
    q_prep = torch.empty_like(bench.base.q)
    qpp, qop = ctypes.c_void_p(bench.base.q.data_ptr()), ctypes.c_void_p(q_prep.data_ptr())
    cpp, spp = ctypes.c_void_p(cos_d.data_ptr()), ctypes.c_void_p(sin_d.data_ptr())

    def prep(i, st):
        rc = L.idx_prep_query(qpp, cpp, spp, prob.rows, 64, 0, qop, ctypes.c_void_p(st))
        if rc:
            raise idx.IdxError(rc, "idx_prep_query")

    us_prep = stream_time(torch, stream, prep, args.steps, args.warmup)

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    key_rows = int(prob.n_keys.astype(np.int64).sum())
    abytes = algorithmic_bytes(prob.n_keys.tolist(), prob.num_pages, prob.rows, prob.k)
    aflops = 2.0 * 64 * 128 * key_rows
    dur_s = us_call * 1e-6
    flops_rate = aflops / dur_s / 1e12
    bytes_rate = abytes / dur_s / 1e9
    score_rate = aflops / (score["median"] * 1e-6) / 1e12
    workload = (f"{args.config}: {prob.num_req} request(s), {prob.rows} rows, n_keys "
                f"{int(prob.n_keys.min())}..{int(prob.n_keys.max())}, H=64, D=128, page 64, k={prob.k}, "
                f"FP8-E4M3 keys + f32 scales, bf16 q and w")
    traffic = measured_traffic(build_hash[:16], args.config)

    out = {
        "metric": "us per score+top-2048 call (4 rows, 128K keys); keys*rows/s; % roofline",
        "value": key_rows / dur_s,
        "unit": "keys*rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": us_call * 1e-3,
        "us_per_call": us_call,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; the workload recipe in workloads/synth.py)",
        "config": {"workload": workload, "key_rows": key_rows, "rotate_copies": bench.copies,
                   "entry_point": "idx_score_topk (score_kernel<8> then select_kernel on one stream)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "dtype": "bf16", "achieved": flops_rate, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops_rate / BF16_PEAK_TFLOPS,
                     "traffic": traffic, "kernel": "one idx_score_topk call (score_kernel<8> + select_kernel)",
                     "algorithmic_flops_per_launch": aflops},
        "roofline_score_kernel": {"bound": "mfma", "dtype": "bf16", "achieved": score_rate,
                                  "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": score_rate / BF16_PEAK_TFLOPS, "kernel": "score_kernel<8> (idx_score)",
                                  "us_per_launch": score["median"]},
        "roofline_hbm": {"bound": "hbm", "achieved": bytes_rate, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bytes_rate / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": abytes},
        "roofline_fp8_context": {"achieved": flops_rate, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": flops_rate / FP8_PEAK_TFLOPS},
        "timing": {"mode": "hipGraph replays of K calls, median over trials",
                   "trials_per_pass": args.trials, "passes": args.passes,
                   "fused_us": fused, "score_only_us": score,
                   "stream_us_per_call": us_stream, "stream_us_per_score_launch": us_stream_score},
        "prep_query": {"entry_point": "idx_prep_query (RoPE on 64 of 128 dims, Hadamard, bf16 out)",
                       "rows": prob.rows, "us_per_launch": us_prep, "timing": "stream, back to back",
                       "bytes_per_launch": prob.rows * 64 * 128 * 2 * 2 + prob.rows * 32 * 4 * 2},
        "library_build_sha256_16": build_hash[:16],
    }

    if not args.no_extra:
        # the 8K-context verify workload, cold: enough calls a trial to cover its copies
        p1, b1, s1, ss1, tr1 = measure("c1", 512, args.warmup)
        f1, sc1 = summary(tr1["fused"]), summary(tr1["score"])
        kr1 = int(p1.n_keys.astype(np.int64).sum())
        out["extra"] = {"c1": {
            "workload": "c1: 1 request, 4 verify rows over an 8,192-key context (8,189..8,192 keys), k=2048",
            "us_per_call": f1["median"], "keys_rows_per_s": kr1 / (f1["median"] * 1e-6),
            "score_only_us": sc1["median"], "fused_us": f1, "stream_us_per_call": s1,
            "rotate_copies": b1.copies, "calls_per_trial": 512,
            "frac_bf16": 2.0 * 64 * 128 * kr1 / (f1["median"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}}
        del b1

    # correctness of the last call and the CPU oracle baseline on the same workload
    if not args.no_cpu:
        from oracle import check as C
        cpu_s, threads, passes, ref, ref_lists = cpu_oracle_baseline(prob, args.cpu_seconds)
        sc = bench.scores.cpu().numpy()
        ls = bench.lists.cpu().numpy()
        worst, exact, missed = 0.0, True, 0
        for r in range(prob.rows):
            n = int(prob.n_keys[r])
            rep = C.check_row(r, sc[r, :n], ls[r], ref[r], n, prob.k)
            worst = max(worst, rep.err_over_max)
            exact = exact and rep.list_ok and rep.score_ok
            missed += rep.missed
        out["cpu_baseline"] = {"value": key_rows / cpu_s, "unit": "keys*rows/s", "cores": threads,
                               "kind": "oracle", "seconds": cpu_s,
                               "sample": f"the whole {args.config} workload ({key_rows} key*rows): f64 gather, "
                                         f"decode, scores (page blocks of each row on a pool of {threads} "
                                         f"threads) and full-sort selection; mean of {passes} passes",
                               "host_cpu": platform.processor() or platform.machine(),
                               "host_cores_available": len(os.sched_getaffinity(0))}
        out["check"] = {"max_err_over_M": worst, "lists_exact_and_scores_in_bound": bool(exact),
                        "missed_vs_f64_topk": int(missed),
                        "ref_lists_sha256_16": hashlib.sha256(ref_lists.tobytes()).hexdigest()[:16]}
    print(json.dumps(out))


if __name__ == "__main__":
    main()
