"""Host-side logic of bench.py (no GPU): the one-GPU guard, the reader of
the committed HBM-traffic counter summaries and the CPU-baseline worker."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _summary(tmp_path, sha, bytes_):
    p = tmp_path / "traffic.txt"
    p.write_text("# header: comment lines are skipped\n"
                 f"kernel: k_4over6_rows\nkernel_src_sha256_16: {sha}\n"
                 f"fetch_scale: 1.99996\nhbm_bytes_per_launch: {bytes_}\n")
    return str(p)


def test_traffic_read_only_for_the_current_kernel_source(tmp_path):
    for w in bench.TRAFFIC:
        assert bench.read_traffic(w, _summary(tmp_path, bench.src_hash(w), "151235333")) == 151235333
        assert bench.read_traffic(w, _summary(tmp_path, "0" * 16, "151235333")) is None
        assert bench.read_traffic(w, str(tmp_path / "absent.txt")) is None


def test_source_hash_covers_the_kernel_and_its_headers():
    for w, (f, srcs) in bench.TRAFFIC.items():
        assert f.startswith("traffic_") and f.endswith(".txt")
        for s in srcs:
            assert os.path.exists(os.path.join(bench.CSRC, s)), s
        h = bench.src_hash(w)
        assert len(h) == 16 and int(h, 16) >= 0 and h == bench.src_hash(w)
    assert bench.METRIC in bench.TRAFFIC


def test_cpu_baseline_worker_runs_the_oracle():
    import numpy as np
    import workloads

    x = workloads.act_rows_input((4, 256))
    assert bench._cpu_task(x, "mae") == 4 * 256
