"""Host-side pieces of bench.py that need no GPU: the one-GPU refusal and
the bounded oracle sampling used for the CPU baselines."""
import os
import subprocess
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and says so,
    before anything touches a device."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_sampled_oracle_sizes_and_scales():
    """The sample grows from a probe toward the time budget, never past the
    workload, and the full-size estimate scales the sample's time by
    full_items / n."""
    calls = []

    def run(n):
        calls.append(n)
        time.sleep(0.002 * n)

    r = bench.sampled_oracle(run, 100, 1e9, 100, "gflops", "the first %d items", budget_s=0.1)
    n = calls[-1]
    assert 8 <= n <= 100
    assert r["sample"] == "the first %d items" % n
    assert r["full_s_estimate"] == pytest.approx(r["seconds"] * 100 / n, rel=0.05, abs=0.01)
    assert r["gflops"] == pytest.approx(n / r["seconds"], rel=0.05)
    assert r["cores"] >= 1
    # a workload smaller than the probe is sampled whole
    calls.clear()
    r = bench.sampled_oracle(run, 3, 1.0, 3, "gflops", "%d", budget_s=0.01)
    assert max(calls) == 3 and r["full_s_estimate"] == pytest.approx(r["seconds"], rel=0.05, abs=0.01)
