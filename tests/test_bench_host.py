"""Host-side logic of bench.py (no GPU): the one-GPU guard, the reader of
the committed HBM-traffic counter summary and the percentile helper."""
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


def test_traffic_read_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, bench.src_hash(), "151235333"))
    assert bench.read_traffic(150470656) == 151235333
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _summary(tmp_path, "0" * 16, "151235333"))
    assert bench.read_traffic(150470656) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.read_traffic(150470656) is None


def test_source_hash_covers_the_kernel_and_its_headers():
    h = bench.src_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert h == bench.src_hash()


def test_percentile_is_nearest_rank():
    v = [7.0, 1.0, 3.0, 9.0, 5.0]
    assert bench.percentile(v, 0) == 1.0
    assert bench.percentile(v, 50) == 5.0
    assert bench.percentile(v, 100) == 9.0
    assert bench.percentile(list(range(101)), 10) == 10
    assert bench.percentile(list(range(101)), 90) == 90
    assert bench.percentile([4.0], 90) == 4.0
