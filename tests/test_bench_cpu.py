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


def test_digest_ignores_comments_and_layout_not_code():
    a = "int f(int x) { return x + 1; } // one\n/* two */"
    b = "int f(int x) {\n  // another comment\n  return x + 1;\n}"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_tokens(a) == bench.code_tokens(b) != bench.code_tokens(c)
    s = 'const char* p = "a // b /* c */"; char q = \'"\'; char r = \'\\\'\';'
    assert bench.code_tokens(s) == s


def test_traffic_only_for_the_sources_it_was_taken_on(monkeypatch):
    """Counters are reported for the sources they were taken on and for no
    other: the committed summary names its source digest."""
    vals = {}
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: vals["source_digest"])
    covered = [k for k in bench.GEMM_KINDS if f"hbm_bytes_per_launch.{k}" in vals]
    assert covered
    for kind in covered:
        v = bench.read_traffic(kind)
        assert v is not None and v > 0, kind
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.read_traffic("grad_logits_gemm") is None


def test_cpu_model_and_threads_reported():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
    assert bench.blas_threads() >= 1
