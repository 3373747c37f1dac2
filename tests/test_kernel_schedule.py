"""CPU check of the generated GEMM main loops (gfx950 assembly, compiled here).

Results do not depend on the loop schedule, but speed does, and a small
source change can silently break it: a second LDS object makes the compiler
wait for every direct load before each fragment read; register pressure can
move spills into the loop. For every GEMM kernel this compiles
kernels_bf16.hip to assembly and checks the innermost 128-MFMA loop:
no scratch traffic, the direct loads and fragment reads the design issues per
two MFMA steps, the barriers, and that the only full vmcnt wait is the one
before the barrier (never between a load and the reads of the same step)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "lm_head_linear_amd", "csrc", "kernels_bf16.hip")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="no hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "k.s")
    r = subprocess.run(["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang",
                        "-target-feature", "-Xclang", "-packed-fp32-ops", "-S",
                        "--cuda-device-only", SRC, "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().split("\n")


@pytest.fixture(scope="module")
def loops(asm):
    lines = asm
    res = {}
    starts = [i for i, l in enumerate(lines) if re.match(r"^_ZN4flce12_GLOBAL__N_16k_gemm\S*:", l)]
    for st in starts:
        en = next(i for i in range(st, len(lines)) if lines[i].startswith(".Lfunc_end"))
        body = lines[st:en]
        name = re.match(r"^_ZN4flce12_GLOBAL__N_16k_gemmILi(\d)ELi(\d)ENS0_(\d+)", body[0])
        epi_name = body[0][name.end():name.end() + int(name.group(3))]   # length-prefixed
        # loop headers as the compiler marks them (a backward jump alone can
        # be a block placed out of line)
        labels = {m.group(1): i for i, l in enumerate(body)
                  if (m := re.match(r"^(\.LBB\d+_\d+):.*Loop Header", l))}
        best = None
        for i, l in enumerate(body):
            m = re.search(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", l)
            if m and m.group(1) in labels and labels[m.group(1)] < i:
                a = labels[m.group(1)]
                if sum("v_mfma" in x for x in body[a:i]) >= 128 and (best is None or i - a < best[1] - best[0]):
                    best = (a, i)
        assert best, body[0]
        seg = [l.strip() for l in body[best[0]:best[1]]
               if l.startswith("\t") and not l.startswith("\t;") and not l.startswith("\t.")]
        res[body[0].split(":")[0]] = (int(name.group(1)), int(name.group(2)), epi_name, seg)
    assert len(res) >= 8
    return res


def _innermost_mfma_loops(body):
    """(start, end) of every loop the compiler marks whose body holds at least
    128 MFMAs and contains no smaller such loop."""
    labels = {m.group(1): i for i, l in enumerate(body)
              if (m := re.match(r"^(\.LBB\d+_\d+):.*Loop Header", l))}
    cand = []
    for i, l in enumerate(body):
        m = re.search(r"s_cbranch_\w+\s+(\.LBB\d+_\d+)", l)
        if m and m.group(1) in labels and labels[m.group(1)] < i:
            a = labels[m.group(1)]
            if sum("v_mfma" in x for x in body[a:i]) >= 128:
                cand.append((a, i))
    return [c for c in cand if not any(o != c and c[0] <= o[0] and o[1] <= c[1] for o in cand)]


@pytest.fixture(scope="module")
def pair_loops(asm):
    """The K loops of the two-GEMM kernels (dH tiles, then dW tiles, of one
    backward chunk in one grid), classified by their operand forms."""
    lines = asm
    res = {}
    for st in [i for i, l in enumerate(lines) if re.match(r"^_ZN4flce12_GLOBAL__N_111k_gemm_pair\S*:", l)]:
        en = next(i for i in range(st, len(lines)) if lines[i].startswith(".Lfunc_end"))
        body = lines[st:en]
        segs = []
        for a, i in _innermost_mfma_loops(body):
            seg = [l.strip() for l in body[a:i]
                   if l.startswith("\t") and not l.startswith("\t;") and not l.startswith("\t.")]
            tr = sum(1 for l in seg if "ds_read_b64_tr_b16" in l)
            segs.append(((0, 1) if tr == 32 else (1, 1), seg))
        res[body[0].split(":")[0]] = segs
    assert len(res) >= 4
    return res


def test_pair_kernels_keep_both_loops(pair_loops):
    """Each two-GEMM kernel holds the dH loop (G K-contiguous, W transposed)
    and the dW loop (both transposed), each scheduled like its own kernel;
    with two K segments (float32 gradients: G's hi and lo parts, the last
    template argument 2) each loop twice."""
    for sym, segs in pair_loops.items():
        n = 2 if re.search(r"ELi2EEEv", sym) else 1
        assert sorted(f for f, _ in segs) == [(0, 1)] * n + [(1, 1)] * n, sym
        for (fa, fb), seg in segs:
            _check_loop(sym, fa, fb, seg)


def test_main_loops(loops):
    for sym, (fa, fb, epi, seg) in loops.items():
        _check_loop(sym, fa, fb, seg)


def _check_loop(sym, fa, fb, seg):
    count = lambda p: sum(1 for l in seg if re.match(p, l))
    assert count(r"v_mfma") == 128, sym
    assert count(r"scratch_|buffer_store|buffer_load") == 0, (sym, "spill in the K loop")
    assert count(r"global_load_lds") == 16, sym          # one stage tile (two steps)
    # fragment reads per two steps: 16 ds_read_b128 per N-form operand,
    # 32 transpose reads per T-form operand (8 row blocks of 16 per step)
    reads = (16 if fa == 0 else 32) + (16 if fb == 0 else 32)
    assert count(r"ds_read") == reads, (sym, count(r"ds_read"))
    # a barrier per two steps
    assert count(r"s_barrier") == 1, sym
    # a full vmcnt wait only directly before a barrier
    for i, l in enumerate(seg):
        if re.match(r"s_waitcnt\s+vmcnt\(0\)", l):
            assert any("s_barrier" in x for x in seg[i + 1:i + 3]), (sym, "vmcnt(0) inside a step")
