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


def test_provenance_without_git_metadata(monkeypatch, tmp_path):
    """Without git (the tree copied without .git), the commit comes from the build record, and
    only while the record's source digest matches the sources."""
    import json
    import subprocess as sp
    sys.path.insert(0, ROOT)
    import bench
    from gated_delta_rule_36_amd import build as b

    def no_git(cmd, *a, **k):
        if cmd and cmd[0] == "git":
            raise OSError("no git here")
        return sp.run(cmd, *a, **k)

    monkeypatch.setattr(sp, "run", no_git)
    rec = tmp_path / "build_info.json"
    monkeypatch.setattr(b, "BUILD_INFO", str(rec))
    assert bench.provenance()["git_sha"] is None  # no record
    rec.write_text(json.dumps({"git_sha": "abc123", "library_sources_committed": True,
                               "source_sha256": b.source_digest()}))
    p = bench.provenance()
    assert p["git_sha"] == "abc123" and p["git_sha_from"] == "build record"
    rec.write_text(json.dumps({"git_sha": "abc123", "library_sources_committed": True,
                               "source_sha256": "0" * 16}))
    assert bench.provenance()["git_sha"] is None  # sources changed since that build
