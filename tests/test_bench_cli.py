"""bench.py's command line on the host: it runs on one GPU and refuses more before touching
any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_counts_each_token_once():
    """The CPU baseline shards one sequence's heads over several processes; the tokens it
    reports are B*T, not B*T times the number of head blocks."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    rng = np.random.default_rng(0)
    B, T, H, d = 1, 8, 4, 3
    x = {n: rng.normal(size=(B, T, H, d)) * (0.1 if n == "g" else 1.0) for n in bench.NAMES}
    x["g"] = -np.abs(x["g"])
    r, parity = bench.cpu_baseline(x, workers=2)
    assert parity is None
    assert r["tokens"] == B * T
    assert r["cores"] == 2
