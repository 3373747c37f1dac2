"""Build libflce.so (HIP kernels for gfx950 + the C-ABI) in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflce.so")

HIP_SOURCES = ["flce_api.hip", "kernels_common.hip", "kernels_bf16.hip", "kernels_f32.hip"]
CXX_SOURCES = ["flce_check.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else (shutil.which("hipcc") or "hipcc")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout)
    return r.stdout


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile every source and link libflce.so; always rebuilds. Returns the path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    flags = HIPCC_FLAGS + list(extra_flags or [])
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in CXX_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append((["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
                      "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src),
                      "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
          *[j[1] for j in jobs], "-lrocprofiler-sdk-roctx"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
