"""bench.py's contract checks that need no GPU."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout


def test_traffic_is_tied_to_the_measured_source():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.fetch_traffic()
    # either the committed counter summary matches the current fetch kernel
    # source, or the bench reports no traffic at all
    if t is not None:
        assert t["total_bytes"] == t["read_bytes"] + t["write_bytes"] > 0
