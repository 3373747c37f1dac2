"""CPU checks of the benchmark's host-side contract: it refuses more than one
GPU with a message, it only reports committed traffic counters while every
library source is unchanged, and those counters cover the four GEMMs."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_digest_covers_every_library_source():
    csrc = os.path.join(ROOT, "lm_head_linear_amd", "csrc")
    listed = {os.path.basename(p) for p in bench.KERNEL_SOURCES}
    assert listed == set(os.listdir(csrc)) - {"__pycache__"}


def test_traffic_only_for_the_sources_it_was_taken_on(monkeypatch):
    for kind in bench.GEMM_KINDS:
        v = bench.read_traffic(kind)
        assert v is not None and v > 0, kind
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.read_traffic("grad_logits_gemm") is None
