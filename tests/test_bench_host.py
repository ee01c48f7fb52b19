"""Host-side logic of bench.py: the algorithmic byte count of the benchmark workload, and
the measured-traffic lookup, which only accepts counters taken on the same library."""
import os

import bench
from workloads import make_config


def test_algorithmic_bytes_of_the_benchmark_workload():
    prob = make_config("c2", scale_down=None)
    got = bench.algorithmic_bytes(prob.n_keys.tolist(), prob.num_pages, prob.rows, prob.k)
    # keys 131,072 x 128 B + scales 131,072 x 4 B + page table 2,048 x 4 B + q 4 x 16 KiB
    # + w 4 x 128 B + n_keys 16 B + scores (131,069..131,072 keys) x 4 B + lists 4 x 2,048 x 4 B
    want = 131072 * 128 + 131072 * 4 + 2048 * 4 + 4 * 16384 + 4 * 128 + 16 + 4 * (4 * 131072 - 6) + 4 * 2048 * 4
    assert got == want == 19505656


def test_measured_traffic_is_keyed_by_the_library_build():
    path = os.path.join(bench.ROOT, "profiles", "score_select_c2_traffic.txt")
    fields = dict(ln.split(":", 1) for ln in open(path).read().splitlines() if ln and not ln.startswith("#"))
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    h = fields["library_build_sha256_16"]
    assert bench.measured_traffic(h, "c2") == int(fields["hbm_bytes_per_launch"])
    assert int(fields["hbm_bytes_per_launch"]) == int(fields["fetch_bytes_per_launch"]) + int(fields["write_bytes_per_launch"])
    assert bench.measured_traffic("0" * 16, "c2") is None
    assert bench.measured_traffic(h, "c1") is None


def test_bench_refuses_more_than_one_gpu():
    """--gpus above 1 exits (status 2) before touching a GPU, with a one-line JSON message."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
