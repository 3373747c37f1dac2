"""Every global address the bf16 GEMM kernels load stays inside its buffer.

Builds tests/csrc/gemm_bounds.cpp against the kernels' own index header and
the library's planner (host code only) and runs it over ragged and full-size
shapes: every launch, workgroup, wave, lane and load (first and last full K
tile, plus the partial tail tile), and that the tile raster is a bijection.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gemm_loads_in_bounds(tmp_path):
    gpp = shutil.which("g++")
    if gpp is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "gemm_bounds")
    r = subprocess.run([gpp, "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "csrc", "gemm_bounds.cpp"),
                        os.path.join(ROOT, "lm_head_linear_amd", "csrc", "flce_check.cpp"),
                        "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ)
    env.pop("FLCE_VCHUNK", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr
    assert "all loads in bounds" in r.stdout
