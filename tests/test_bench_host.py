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


def test_traffic_counters_follow_their_sources():
    """A stored counter reading counts only for its workload and kernel and while the
    kernel's sources hash to the value it was taken on."""
    e = {"workload": "1.7b-bf16", "kernel": "gate_up", "sha256": bench.source_sha(bench.GEMM_SOURCES),
         "fetch_kib": 34365.5, "write_kib": 1344.0}
    t = bench.counter_traffic(e, "1.7b-bf16", "gate_up")
    assert t == pytest.approx((34365.5 * bench.FETCH_FACTOR + 1344.0 * bench.WRITE_FACTOR) * 1024.0)
    assert bench.counter_traffic(e, "8b-bf16-tree", "gate_up") is None
    assert bench.counter_traffic(e, "1.7b-bf16", "down") is None
    assert bench.counter_traffic(dict(e, sha256="0" * 64), "1.7b-bf16", "gate_up") is None
    for entry in bench.TRAFFIC:     # stored entries name a known kernel kind
        assert entry["kernel"] in bench.KERNEL_SOURCES


def test_pass_bytes_match_the_configs():
    """Algorithmic bytes per pass of the 1.7B and 8B-tree workloads: weights once, KV read
    and written, fp32 logits of the acceptance rows (plus the fp32 norm gains and the
    gathered embedding rows, under 0.01 %)."""
    from synth.configs import WORKLOADS
    c2, c3 = WORKLOADS["1.7b-bf16"](), WORKLOADS["8b-bf16-tree"]()
    b2 = bench.pass_bytes(c2.shape, c2.T, c2.R, list(c2.ctx))
    b3 = bench.pass_bytes(c3.shape, c3.T, c3.R, list(c3.ctx))
    assert b2 == pytest.approx(4_239_630_336, rel=1e-4)
    assert b3 == pytest.approx(16_379_786_752, rel=1e-4)


def test_launch_work_of_the_decoder_kinds():
    from synth.configs import SHAPE_1P7B
    sh = SHAPE_1P7B
    w = bench.launch_work(sh, 1, 41, 17, [4096], None, "lm")
    assert w["gate_up"][0] == 2 * 8192 * 2048 * 2 + 41 * 2048 * 4 + 41 * 8192 * 4
    assert w["gate_up"][1] == 2.0 * 41 * 16384 * 2048
    # attention: every query row of a chain sees C cached keys plus itself and its predecessors
    assert w["attention"][1] == 4.0 * 32 * 64 * (41 * 4096 + 41 * 42 // 2)
    assert bench.attn_visible_keys(3, 10, [-1, 0, 0]) == 3 * 10 + 1 + 2 + 2


def test_step_distribution_reports_median_and_tails():
    """Per-step times of a timed region: median, 10th and 90th percentile, count."""
    d = bench.step_distribution([4.0, 1.0, 3.0, 2.0, 5.0, 10.0, 6.0, 8.0, 7.0, 9.0])
    assert d == {"median": 5.5, "p10": pytest.approx(1.9), "p90": pytest.approx(9.1), "n": 10}
    one = bench.step_distribution([2.5])
    assert one["median"] == one["p10"] == one["p90"] == 2.5 and one["n"] == 1
