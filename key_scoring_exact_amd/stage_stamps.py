"""Stage timings of one idx_score_topk call from in-kernel timestamps.

Builds a second copy of the library with -DIDX_STAMPS (libidx_stamps.so, beside
libidx.so), in which thread 0 of every workgroup writes the GPU's 100 MHz real-time
counter at the end of each stage into the workspace.  Runs the call `--calls` times
over rotating key-cache copies (cold keys, as the benchmark), reads the stamps after
each call and prints, per stage, the median over calls of the median over workgroups:
the time from the call's first scoring workgroup start, and the stage's own duration.

    python -m key_scoring_exact_amd.stage_stamps [--config c2] [--calls 50]

Stages of the scoring launch (per workgroup): 1 key counts and page ids in registers;
2 the first key page in LDS; 3 MFMA loop and epilogue done; 4 score stores issued; 5
candidate publication done (wave 0's row).  Of the selection launch (per row): 0 start;
1 chunk headers reduced (or, for a row selected from all its scores, those scores in
LDS); 2 candidates gathered; 5 keys in registers; 6 linear histogram built; 7 bin of the
k-th key found; 3 k-th key resolved; 4 list written.  A stage a row does not pass is
left out of that row's figures.
"""
from __future__ import annotations

import argparse
import ctypes
import math
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
STAMPS_LIB = os.path.join(HERE, "libidx_stamps.so")
SLOTS, SELECT0 = 16, 8192
TICK_US = 0.01                              # 100 MHz counter

SCORE_STAGES = [(1, "key counts, page ids, queries loaded"), (2, "first key page in LDS"),
                (3, "MFMA loop and epilogue done"), (4, "score stores issued"),
                (5, "publication done (wave 0)")]
SELECT_STAGES = [(0, "selection start"), (1, "chunk headers reduced, or the row's scores in LDS"),
                 (2, "candidates gathered"), (5, "keys in registers"), (6, "linear histogram"),
                 (7, "bin of the k-th key found"), (8, "the bin's keys listed"),
                 (10, "k-th key among them (wave 0)"), (3, "k-th key resolved"),
                 (11, "list places counted (piece-major)"), (12, "list offsets scanned (piece-major)"),
                 (4, "list written")]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", default="c2")
    ap.add_argument("--calls", type=int, default=50)
    ap.add_argument("--rotate-mib", type=int, default=512)
    ap.add_argument("--no-build", action="store_true")
    args = ap.parse_args(argv)

    import numpy as np
    import torch

    sys.path.insert(0, os.path.dirname(HERE))
    from key_scoring_exact_amd import DeviceProblem, _lib
    from key_scoring_exact_amd import build as B
    from workloads import make_config

    if not args.no_build or not os.path.exists(STAMPS_LIB):
        B.build(out=STAMPS_LIB, extra_flags=["-DIDX_STAMPS"])
    L = _lib.load_file(STAMPS_LIB)
    torch.cuda.set_device(0)
    prob = make_config(args.config)
    bounds = [int(prob.n_keys[a:b].max()) for a, b in zip(prob.req_indptr[:-1], prob.req_indptr[1:])]
    base = DeviceProblem.from_arrays(prob.q, prob.w, prob.k_cache, prob.k_scale, prob.page_table, prob.n_keys,
                                     prob.req_indptr, max_keys=prob.max_keys, req_max_keys=bounds)
    copy_bytes = base.k_cache.numel() + base.k_scale.numel() * 4
    copies = max(1, math.ceil(args.rotate_mib * (1 << 20) / copy_bytes))
    probs = [base] + [DeviceProblem(q=base.q, w=base.w, k_cache=base.k_cache.clone(), k_scale=base.k_scale.clone(),
                                    page_table=base.page_table, n_keys=base.n_keys, req_indptr=base.req_indptr,
                                    max_keys=base.max_keys, req_max_keys=base.req_max_keys)
                     for _ in range(copies - 1)]
    structs = [p.struct() for p in probs]
    need = ctypes.c_size_t(0)
    assert L.idx_workspace_bytes(prob.rows, base.max_keys, prob.k, ctypes.byref(need)) == 0
    nbytes = need.value
    buf = torch.zeros(nbytes + 256, dtype=torch.uint8, device="cuda")
    off = (-buf.data_ptr()) % 256
    wsp = buf.data_ptr() + off
    st = torch.cuda.current_stream().cuda_stream
    assert L.idx_workspace_init(ctypes.c_void_p(wsp), nbytes, ctypes.c_void_p(st)) == 0
    scores = torch.empty((prob.rows, base.max_keys), dtype=torch.float32, device="cuda")
    lists = torch.empty((prob.rows, prob.k), dtype=torch.int32, device="cuda")
    area = SLOTS * 8 * (SELECT0 + 4 * 256)
    stamps_off = off + nbytes - area            # the stamp area ends the workspace

    def call(i):
        s, _ = structs[i % copies]
        rc = L.idx_score_topk(ctypes.byref(s), prob.k, ctypes.c_void_p(scores.data_ptr()), scores.shape[1],
                              ctypes.c_void_p(lists.data_ptr()), ctypes.c_void_p(wsp), nbytes, ctypes.c_void_p(st))
        assert rc == 0, rc

    for i in range(10):
        call(i)
    torch.cuda.synchronize()
    per_stage = {("score", s): [] for s, _ in SCORE_STAGES}
    per_stage.update({("select", s): [] for s, _ in SELECT_STAGES})
    durs = {("score", s): [] for s, _ in SCORE_STAGES}
    durs.update({("select", s): [] for s, _ in SELECT_STAGES})
    total = []
    for i in range(args.calls):
        buf[stamps_off: stamps_off + area].zero_()
        call(i)
        torch.cuda.synchronize()
        rec = buf[stamps_off: stamps_off + area].cpu().numpy().view(np.uint64).reshape(-1, SLOTS).astype(np.int64)
        sc = rec[:SELECT0]
        sc = sc[sc[:, 0] > 0]
        se = rec[SELECT0:]
        se = se[se[:, 0] > 0]
        t0 = sc[:, 0].min()
        for s, _ in SCORE_STAGES:
            ok = sc[:, s] > 0
            if ok.any():
                per_stage[("score", s)].append(float(np.median(sc[ok, s] - t0)))
                prev = s - 1
                durs[("score", s)].append(float(np.median(sc[ok, s] - sc[ok, prev])))
        order = [p for p, _ in SELECT_STAGES]
        for idx_s, (s, _) in enumerate(SELECT_STAGES):
            ok = se[:, s] > 0
            if not ok.any():
                continue
            per_stage[("select", s)].append(float(np.median(se[ok, s] - t0)))
            if s == 0:
                durs[("select", s)].append(float(np.median(se[ok, 0] - sc[:, 5][sc[:, 5] > 0].max())))
                continue
            # the stage's duration from the latest earlier stage the row passed
            prev = np.zeros(len(se), dtype=np.int64)
            for p in order[:idx_s]:
                prev = np.where(se[:, p] > 0, se[:, p], prev)
            durs[("select", s)].append(float(np.median(se[ok, s] - prev[ok])))
        total.append(float(se[:, 4].max() - t0) if len(se) else float("nan"))
    print(f"# stage stamps, {args.config}: {prob.rows} rows, n_keys {int(prob.n_keys.min())}..{int(prob.n_keys.max())}, "
          f"{args.calls} calls over {copies} key-cache copies; median over calls of the median over workgroups, us")
    print("| launch | stage | ends at (from first scoring workgroup start) | takes (per workgroup) |")
    print("|---|---|---|---|")
    for s, name in SCORE_STAGES:
        print(f"| scoring | {name} | {statistics.median(per_stage[('score', s)]) * TICK_US:.2f} | "
              f"{statistics.median(durs[('score', s)]) * TICK_US:.2f} |")
    for s, name in SELECT_STAGES:
        if not per_stage[("select", s)]:
            continue
        lab = name if s else name + " (after the last scoring workgroup's stamp 5)"
        print(f"| selection | {lab} | {statistics.median(per_stage[('select', s)]) * TICK_US:.2f} | "
              f"{statistics.median(durs[('select', s)]) * TICK_US:.2f} |")
    print(f"| call | first scoring start to last list written | {statistics.median(total) * TICK_US:.2f} | |")


if __name__ == "__main__":
    main()
