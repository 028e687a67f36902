"""Host-side checks of bench.py: the multi-GPU refusal and the traffic figure's
provenance (the counter summary is only reported for the workload and the GEMM
source it was taken on)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_traffic_only_for_its_workload():
    path = os.path.join(ROOT, "profiles", f"expert_gemm_{bench.TRAFFIC_WORKLOAD}_traffic.txt")
    if not os.path.exists(path):
        pytest.skip("no counter summary committed")
    recorded = [l.split("=", 1)[1].strip() for l in open(path) if l.startswith("source_sha256_16=")]
    v = bench.read_traffic("expert_up", bench.TRAFFIC_WORKLOAD)
    if recorded and recorded[0] == bench.kernel_source_hash():
        assert v is not None and v > 0
    else:
        assert v is None
    for other in ("many_expert_train", "mixtral_8x7b", "deepseek_v3"):
        assert bench.read_traffic("expert_up", other) is None
        assert bench.read_traffic("expert_down", other) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)
