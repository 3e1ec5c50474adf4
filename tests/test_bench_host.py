"""Host-side pieces of bench.py that need no GPU: the one-GPU refusal and
the bounded oracle sampling used for the CPU baselines, and the per-XCD
grouping of the clock-hook stamps."""
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


def test_per_xcd_groups_units_by_slot():
    """bench.per_xcd: unit u runs in slot u % grid, slots [32x, 32x + 32) of a
    256 grid on XCD x; the clock is cycles over real time (100 MHz ticks)."""
    import numpy as np

    grid, units = 256, 512
    st = np.zeros((units, 6))
    for u in range(units):
        x = (u % grid) // 32
        start = 0.0 if u < grid else 1000.0 + 10 * x
        st[u, 0], st[u, 1] = start, start + 1000.0          # 10 us each
        st[u, 2], st[u, 3] = 0.0, (1600.0 + 25 * x) * 10.0  # cycles over 10 us
    out = bench.per_xcd(st, grid)
    assert out["sclk_mhz"] == [1600.0 + 25 * x for x in range(8)]
    assert out["last_end_us"] == [20.0 + 0.1 * x for x in range(8)]
    assert bench.per_xcd(st, 250) is None
