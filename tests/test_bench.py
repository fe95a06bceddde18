"""Host-side parts of bench.py's contract (no GPU needed)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_only_for_its_workload_and_kernel_source(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    name = t["workload"].split(" ")[0]
    if t["gemm_source_sha256_16"] == bench.gemm_source_hash():
        assert bench.measured_traffic(name) == t["bytes_per_launch"]
    assert bench.measured_traffic("attn8b_tw" if name != "attn8b_tw" else "ffn8b_tw") is None
    # counters taken on another version of the kernel are not reported
    stale = dict(t, gemm_source_sha256_16="0" * 16)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic(name) is None
