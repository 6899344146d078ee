"""Host-side logic of bench.py (no GPU): the one-GPU refusal, and the stored HBM
traffic counters, which count only for the kernel sources they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.parametrize("stored,workload,files", [
    (bench.GATE_UP_TRAFFIC, "1.7b-bf16", bench.GEMM_SOURCES),
    (bench.ROW_STATS_TRAFFIC, "sample", bench.SAMPLE_SOURCES),
])
def test_traffic_counters_follow_their_sources(stored, workload, files):
    t = bench.counter_traffic(stored, workload, files)
    if stored["sha256"] != bench.source_sha(files):
        assert t is None          # sources changed since the counters were taken
        return
    assert t == pytest.approx((stored["fetch_kib"] * stored["fetch_factor"]
                               + stored["write_kib"] * stored["write_factor"]) * 1024.0)
    assert bench.counter_traffic(stored, "another-workload", files) is None
    assert bench.counter_traffic(dict(stored, sha256="0" * 64), workload, files) is None
