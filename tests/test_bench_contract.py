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


def test_step_counter_traffic_records_parse():
    # each committed decode-step profile gives the whole step's counter bytes
    # and its algorithmic weight (+ KV) bytes, or nothing once the kernel
    # sources have changed since the counters were taken; the counter bytes
    # cover the weights at least once and the extra traffic (split-K planes,
    # images, partials) stays well below the weights themselves
    for name in ("decode_step_llama3_8b_q4_m32.md", "decode_step_qwen05b_q8_m1.md"):
        rec = bench.step_counter_traffic(name, 1e-3, "test")
        if rec is None:
            continue
        assert rec["algorithmic_bytes_per_step"] <= rec["bytes_per_step"]
        assert rec["bytes_per_step"] <= 1.5 * rec["algorithmic_bytes_per_step"]
        assert abs(rec["gbs"] - rec["bytes_per_step"] / 1e-3 / 1e9) < 1e-6 * rec["gbs"]


def test_kernel_sources_hash_is_stable():
    assert bench.kernel_sources_sha256() == bench.kernel_sources_sha256()
    assert len(bench.kernel_sources_sha256()) == 64
