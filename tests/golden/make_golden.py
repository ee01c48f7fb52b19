"""Write tests/golden/oracle_digests.json from the seeded generators and the CPU oracle.

Run from the repository root:  python tests/golden/make_golden.py
The stored digests pin the generators and the oracle against unintended
change; they are produced by this script only (workloads + oracle).
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import indexer as O  # noqa: E402
from workloads import make_config  # noqa: E402

CASES = [("c0", None), ("c1", 4), ("c3", 16), ("c4a", 32), ("c4c", 32)]


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def case_digests(name, scale_down):
    p = make_config(name, scale_down=scale_down)
    vs = O.scores(p)
    lists = O.topk(p, vs)
    return {
        "inputs": sha(np.concatenate([p.q.view(np.uint8).ravel(), p.w.view(np.uint8).ravel(),
                                      p.k_cache.ravel(), p.k_scale.view(np.uint8).ravel(),
                                      p.page_table.view(np.uint8).ravel(), p.n_keys.view(np.uint8).ravel()])),
        "scores_f32": [sha(v.astype(np.float32)) for v in vs],
        "lists": [sha(lists[r]) for r in range(p.rows)],
    }


def main():
    out = {f"{n}/{s or 1}": case_digests(n, s) for n, s in CASES}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_digests.json")
    with open(path, "w") as f:
        json.dump({"_about": "SHA-256 of seeded inputs and of the CPU oracle's scores (rounded to f32) "
                             "and lists; written by tests/golden/make_golden.py", **out}, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
