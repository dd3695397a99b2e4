"""Host-side logic of bench.py (no GPU): the HBM traffic figure it reports is
taken from the committed counter summary only for the same workload and the
same score-kernel sources, and a request for more than one GPU is refused."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _summary(tmp_path, workload, sha, nbytes="1985557576"):
    p = tmp_path / "traffic.txt"
    p.write_text("# a comment: with a colon\n"
                 "workload: %s\nsource_sha256: %s\nbytes_per_launch: %s\n" % (workload, sha, nbytes))
    return str(p)


def test_traffic_gated_by_workload_and_sources(tmp_path):
    sha = bench.score_source_hash()
    assert len(sha) == 64
    assert bench.measured_traffic(_summary(tmp_path, "pages", sha), "pages") == 1985557576.0
    # another workload, or sources that changed since the counters were taken: no figure
    assert bench.measured_traffic(_summary(tmp_path, "pages", sha), "mid") is None
    assert bench.measured_traffic(_summary(tmp_path, "pages", "0" * 64), "pages") is None
    # a missing file or a malformed value: no figure
    assert bench.measured_traffic(str(tmp_path / "absent.txt"), "pages") is None
    assert bench.measured_traffic(_summary(tmp_path, "pages", sha, "n/a"), "pages") is None


def test_committed_summary_parses():
    """The committed summary names the pages workload and a positive byte count (its hash
    matches only while the kernel sources are those the counters were taken on)."""
    path = os.path.join(ROOT, "profiles", "score_kernel_pages_traffic.txt")
    kv = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert kv["workload"] == "pages" and len(kv["source_sha256"]) == 64
    assert float(kv["bytes_per_launch"]) > 0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
