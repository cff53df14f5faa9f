"""bench.py's command-line contract that needs no GPU: one GPU only, and the
HBM traffic it reports comes from counters taken on the current kernels."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_counters_match_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    t = bench.measured_traffic()
    if t is None:
        pytest.skip("kernel sources changed since the counters were taken (bench reports traffic: null)")
    # one 8K batch-1 call: 17.30 MB of K/V codes and steps; the counted bytes
    # include the query, tables, partials and the merge's reads
    assert 17_301_504 <= t <= 1.1 * 17_301_504
