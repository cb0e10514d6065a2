"""Host-side checks of bench.py's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_traffic_record_parses():
    # the committed counter summary gives the chunk kernel's HBM bytes per
    # launch and that launch's algorithmic bytes, or nothing once the attention
    # source has changed since the counters were taken
    traffic, alg = bench.counter_traffic()
    assert (traffic is None) == (alg is None)
    if traffic is not None:
        assert 0.95 * alg <= traffic <= 1.10 * alg
