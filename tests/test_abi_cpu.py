"""CPU-only tests of the C-ABI library: it loads, exports every declared symbol,
and its synchronous checks and workspace planner behave as documented. No GPU
compute call is made here (pointers are fake integers, never dereferenced)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")


@pytest.fixture(scope="module")
def lib():
    from lm_head_linear_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from lm_head_linear_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("flce_forward_backward", "flce_workspace_size", "flce_check_args",
                 "flce_status_string"):
        assert must in names


def test_every_declared_symbol_is_exported(lib):
    from lm_head_linear_amd import _lib
    names = declared_functions()
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature in the binding"
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                             text=True).stdout
        exported = set(re.findall(r"\bT\s+(\w+)", out))
        for n in names:
            assert n in exported, n


def test_status_strings(lib):
    for code in range(7):
        s = lib.flce_status_string(code).decode()
        assert s.startswith("FLCE_")
    assert "unknown" in lib.flce_status_string(99).decode()


GiB = 1 << 30
MiB = 1 << 20


@pytest.mark.parametrize("N,H,V,limit", [
    (8192, 4096, 131072, 512 * MiB),      # N*V*4/8 for the large-vocab case
    (8192, 3584, 256000, 1 * GiB),        # softcapped case
    (16384, 4096, 131072, 1 * GiB),       # the [2, 8192, 131072] case
])
def test_workspace_far_below_logits(lib, N, H, V, limit):
    """Extra memory stays at or below 1/8 of the float32 logits it avoids.

    Modalities PR 464, "Memory note": a [2, 8192, 131072] float32 logit tensor
    is 8 GiB; the workspace here is bounded by 1/8 of N*V*4.
    """
    ws = lib.flce_workspace_size(N, H, V, 1)
    assert 0 < ws <= limit
    assert ws <= N * V * 4 // 8
    if (N, V) == (16384, 131072):
        assert N * V * 4 == 8 * GiB


def test_workspace_invalid_sizes(lib):
    assert lib.flce_workspace_size(-1, 8, 8, 1) == 0
    assert lib.flce_workspace_size(8, 0, 8, 1) == 0
    assert lib.flce_workspace_size(8, 8, 0, 1) == 0
    assert lib.flce_workspace_size(8, 8, 8, 7) == 0
    assert lib.flce_workspace_size(0, 8, 8, 1) > 0


def test_kept_chunks_plan(lib):
    """Chunks whose logit gradient comes from the forward's kept probabilities:
    chunk 0 alone (in the workspace) when dW is added to; otherwise chunks
    0 .. m-1 one after another at the top of dW, each past the rows of chunks
    0 .. j, and chunk m in the workspace, for the largest m < 4 that fits.
    Large-vocab: dW 1 GiB, rows of a chunk 128 MiB, G 256 MiB: chunks 0, 1, 2
    at 256, 512, 768 MiB (past 128, 256, 384 MiB of rows); four in dW would put
    chunk 0 at 0."""
    assert lib.flce_kept_chunks(8192, 4096, 131072, 1, 0) == 4
    assert lib.flce_kept_chunks(8192, 4096, 131072, 1, 1) == 1     # dW added to
    # softcapped: rows 218.75 MiB, G 500 MiB of 1750 MiB: chunks 0-2 at 250,
    # 750, 1250 MiB, past 218.75, 437.5, 656.25 MiB of rows
    assert lib.flce_kept_chunks(8192, 3584, 256000, 1, 0) == 4
    # long: chunk 16384 rows (128 MiB of dW each), G 512 MiB: chunk 0 at 512 MiB;
    # two in dW would put chunk 0 at 0
    assert lib.flce_kept_chunks(16384, 4096, 131072, 1, 0) == 2
    # a long micro-batch: 4 chunks of 32768 rows (256 MiB each), G 256 MiB: chunks
    # 0-2 at 256, 512, 768 MiB, chunk 3 in the workspace: nothing recomputed
    assert lib.flce_kept_chunks(4096, 4096, 131072, 1, 0) == 4
    assert lib.flce_kept_chunks(2048, 1024, 32000, 1, 0) == 1      # one chunk
    assert lib.flce_kept_chunks(32, 64, 1024, 0, 0) == 0           # float32: recomputed
    assert lib.flce_kept_chunks(0, 64, 1024, 1, 0) == 0
    assert lib.flce_kept_chunks(8, 8, 0, 1, 0) == 0


def test_vocab_chunk_plan(lib):
    """G's chunk takes up to 2^27 elements, or N V 4 / 16 bytes when that is
    more, and the vocabulary is split into equal chunks (a multiple of the
    tile each)."""
    assert lib.flce_vocab_chunk(8192, 4096, 131072, 1) == 16384      # 2^27 elements
    assert lib.flce_vocab_chunk(16384, 4096, 131072, 1) == 16384     # N V / 8 elements
    assert lib.flce_vocab_chunk(8192, 3584, 256000, 1) == 32000      # 8 chunks of 125 tiles
    assert lib.flce_vocab_chunk(2048, 1024, 32000, 1) == 32000       # one chunk
    assert lib.flce_vocab_chunk(32, 64, 1024, 0) == 1024
    # balanced: 3 chunks of 2^27 / 8192 = 16384 rows would leave a short last
    # one; 40000 rows go in 3 chunks of 13568
    assert lib.flce_vocab_chunk(8192, 1024, 40000, 1) == 13568
    for N, V in [(8192, 131072), (8192, 256000), (16384, 131072), (4000, 50257), (777, 1500)]:
        c = lib.flce_vocab_chunk(N, 1024, V, 1)
        n = -(-V // c)
        assert c % 256 == 0 and 256 <= c <= -(-V // 256) * 256
        assert c * ((N + 7) // 8 * 8) <= max(1 << 27, N // 4 * V // 2)
        assert V - (n - 1) * c > 0 and c - (V - (n - 1) * c) < 256 * n


# -------------------------------------------------------------- check_args
A16 = 1 << 20          # fake, 256-aligned "device" addresses (never dereferenced)


def _args(**kw):
    N, H, V = kw.get("N", 64), kw.get("H", 64), kw.get("V", 128)
    dtype = kw.get("dtype", 1)
    base = dict(h=A16, W=A16 * 64, labels=A16 * 128, N=N, H=H, V=V, ignore=-100, softcap=0.0,
                red=0, T=0, loss=A16 * 129, nt=A16 * 130, dH=A16 * 256, dW=A16 * 512,
                stream=None, dtype=dtype, mb=1.0, acc=0, ws=A16 * 1024, wsb=1 << 40,
                status=None, lse=None)
    base.update({k: v for k, v in kw.items() if k in base})
    return [base[k] for k in ("h", "W", "labels", "N", "H", "V", "ignore", "softcap", "red",
                              "T", "loss", "nt", "dH", "dW", "stream", "dtype", "mb", "acc",
                              "ws", "wsb", "status", "lse")]


def test_check_args_ok(lib):
    assert lib.flce_check_args(*_args()) == 0
    assert lib.flce_check_args(*_args(dtype=0, H=3)) == 0      # fp32: any H
    for mb in (0.0, -0.0, 0.25, 1.0, 3.0):                     # any finite scale >= 0
        assert lib.flce_check_args(*_args(mb=mb)) == 0, mb


def test_negative_micro_batch_scale_rejected_by_every_entry(lib):
    """The token-weighted micro-batch scale (twinkle PR 335, "PR information",
    item 2) is a fraction of tokens, never negative: every entry point's
    checks refuse a negative one before any launch."""
    a = _args(mb=-0.5)
    assert lib.flce_check_args(*a) == 1
    assert lib.flce_check_args_ex(*a, 1) == 1
    assert lib.flce_check_args_ex(*a, 0) == 1
    assert lib.flce_check_args_nr(*a, 0) == 1
    fw = [a[i] for i in range(22) if i not in (12, 13, 17)]   # no dH, dW, accumulate_dW
    assert lib.flce_forward_check_args(*fw) == 1
    assert lib.flce_forward_logits_check_args(*fw, A16 * 2048, 128, 0) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 1), (dict(H=0), 1), (dict(V=0), 1),
    (dict(red=2), 1), (dict(dtype=5), 1),
    (dict(softcap=-1.0), 1), (dict(softcap=float("inf")), 1), (dict(softcap=float("nan")), 1),
    (dict(mb=float("nan")), 1), (dict(mb=float("inf")), 1),
    (dict(mb=-0.5), 1), (dict(mb=-1e-30), 1),      # the micro-batch scale is a token fraction
    (dict(red=1, T=10), 1),
    (dict(h=None), 1), (dict(W=None), 1), (dict(labels=None), 1), (dict(loss=None), 1),
    (dict(nt=None), 1), (dict(dH=None), 1), (dict(dW=None), 1),
    (dict(dH=A16), 1),                 # dH aliases h
    (dict(dW=A16 * 64 + 256), 1),      # dW overlaps W
    (dict(dH=A16 * 64), 1),            # dH overlaps W
    (dict(dW=A16), 1),                 # dW overlaps h
    (dict(h=A16 + 8), 2),              # misaligned bf16 matrix
    (dict(ws=None), 3), (dict(ws=A16 * 1024 + 128), 3), (dict(wsb=16), 3),
])
def test_check_args_errors(lib, kw, code):
    assert lib.flce_check_args(*_args(**kw)) == code


def test_odd_hidden_size_runs_padded(lib):
    """bf16 with H % 8 != 0 (the NeMo linear_ce page, "API", puts no limit on
    the hidden size): every entry point accepts it and carves padded copies at
    the width rounded up to 8: W, dW and dH, and h where the tokens are not
    gathered (the logits-returning and allocation-free forwards)."""
    assert lib.flce_check_args(*_args(H=12)) == 0
    assert lib.flce_check_args_ex(*_args(H=12), 0) == 0
    assert lib.flce_check_args_nr(*_args(H=12), 0) == 0
    fw = [x for i, x in enumerate(_args(H=12)) if i not in (12, 13, 17)]
    assert lib.flce_forward_check_args(*fw) == 0
    fws = [x for i, x in enumerate(_args(H=12, wsb=1 << 20)) if i not in (12, 13, 17)]
    assert lib.flce_forward_logits_check_args(*fws, A16 * 2048, 128, 0) == 0
    # the logits entry (no gather, a padded copy of h instead) fits the forward workspace
    fwsz = lib.flce_forward_workspace_size(64, 12, 128, 1)
    fwx = [x for i, x in enumerate(_args(H=12, wsb=fwsz)) if i not in (12, 13, 17)]
    assert lib.flce_forward_logits_check_args(*fwx, A16 * 2048, 128, 0) == 0
    assert lib.flce_check_args(*_args(H=12, dH=A16)) == 1       # argument errors come first
    N, V = 300, 1000
    for H in (1, 100, 4095):
        Hp = -(-H // 8) * 8
        pad_w, pad_g = V * Hp * 2, V * Hp * 2 + N * Hp * 2           # W; dW and dH
        slack = 3 * 256 + N * 8                                      # alignment; hc rows
        extra = lib.flce_workspace_size(N, H, V, 1) - lib.flce_workspace_size(N, Hp, V, 1)
        assert pad_w + pad_g <= extra <= pad_w + pad_g + slack, (H, extra)
        extra = (lib.flce_forward_workspace_size(N, H, V, 1)
                 - lib.flce_forward_workspace_size(N, Hp, V, 1))
        assert pad_w <= extra <= pad_w + slack, (H, extra)
        extra = lib.flce_workspace_size_ex(N, H, V, 1, 0) - lib.flce_workspace_size_ex(N, Hp, V, 1, 0)
        assert pad_w + 2 * pad_g <= extra <= pad_w + 2 * pad_g + slack, (H, extra)
        extra = lib.flce_workspace_size_nr(N, H, V, 1, 0) - lib.flce_workspace_size_nr(N, Hp, V, 1, 0)
        assert pad_w + pad_g <= extra <= pad_w + pad_g + slack, (H, extra)
        assert lib.flce_vocab_chunk(N, H, V, 1) == lib.flce_vocab_chunk(N, Hp, V, 1)
    assert lib.flce_workspace_size(8, 12, 8, 0) == lib.flce_workspace_size(8, 12, 8, 0)  # fp32: as is


def test_check_args_empty_batch(lib):
    # N = 0: h, labels, dH may be NULL
    assert lib.flce_check_args(*_args(N=0, h=None, labels=None, dH=None)) == 0


def test_mean_with_T_rejected_sum_with_T_ok(lib):
    assert lib.flce_check_args(*_args(red=0, T=123)) == 0
    assert lib.flce_check_args(*_args(red=1, T=0)) == 0
    assert lib.flce_check_args(*_args(red=1, T=-5)) == 0


def test_forward_backward_rejects_before_launch(lib):
    """Synchronous errors return before any HIP call, so this runs without a GPU."""
    assert lib.flce_forward_backward(*_args(N=-1)) == 1
    assert lib.flce_forward_backward(*_args(wsb=1)) == 3


def test_python_binding_validation_without_gpu():
    import lm_head_linear_amd as m
    h = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        m.flce_forward_backward(h, W, y)          # CPU tensors: refused, no fallback
    with pytest.raises(ValueError):
        m.FusedLinearCrossEntropy(reduction="avg")
    assert m.micro_batch_scale(3, 12, "mean") == 0.25
    assert m.micro_batch_scale(3, 12, "sum") == 1.0


class _FakeBuf:
    """Stands in for a device tensor in the binding's check wrappers, which
    only read its address and size (never its contents)."""

    def __init__(self, addr, nbytes=0):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def test_python_binding_has_every_abi_name(lib):
    """The binding offers each entry point of the header under its own name."""
    import lm_head_linear_amd as m
    for n in declared_functions():
        assert callable(getattr(m, n, None)), n
        assert n in m.__all__, n


@pytest.mark.parametrize("kw", [dict(), dict(wsb=16), dict(red=1, T=7), dict(dH=None),
                                dict(mb=-0.5)])
def test_python_check_wrappers_match_the_library(lib, kw):
    import lm_head_linear_amd as m
    a = dict(zip(("h", "W", "labels", "N", "H", "V", "ignore", "softcap", "red", "T", "loss",
                  "nt", "dH", "dW", "stream", "dtype", "mb", "acc", "ws", "wsb", "status",
                  "lse"), _args(**kw)))
    f = lambda x: None if x is None else _FakeBuf(x)
    py = dict(N=a["N"], H=a["H"], V=a["V"], ignore_index=a["ignore"], softcap=a["softcap"],
              reduction="mean" if a["red"] == 1 else "sum", num_label_tokens=a["T"] or None,
              loss=f(a["loss"]), num_tokens=f(a["nt"]), dH=f(a["dH"]), dW=f(a["dW"]),
              dtype=torch.bfloat16, mb_scale=a["mb"], workspace=_FakeBuf(a["ws"], a["wsb"]))
    h, W, y = _FakeBuf(a["h"]), _FakeBuf(a["W"]), _FakeBuf(a["labels"])
    assert m.flce_check_args_nr(h, W, y, token_chunk=256, **py) == \
        lib.flce_check_args_nr(*_args(**kw), 256)
    assert m.flce_check_args_ex(h, W, y, grad_dtype=torch.float32, **py) == \
        lib.flce_check_args_ex(*_args(**kw), 0)
    assert m.flce_check_args(h, W, y, **py) == lib.flce_check_args(*_args(**kw))


def test_python_size_and_profile_wrappers_match_the_library(lib):
    import lm_head_linear_amd as m
    bf, f32 = torch.bfloat16, torch.float32
    assert m.flce_workspace_size_ex(8192, 4096, 131072, bf, f32) == \
        lib.flce_workspace_size_ex(8192, 4096, 131072, 1, 0)
    assert m.flce_vocab_chunk_ex(8192, 4096, 131072, bf, f32) == \
        lib.flce_vocab_chunk_ex(8192, 4096, 131072, 1, 0)
    assert m.flce_profile_kinds() == lib.flce_profile_kinds()
    assert m.kernel_kinds()[0] == m.flce_kernel_kind_name(0) == "label_scan"


def test_sanitized_host_checks(tmp_path):
    """flce_check.cpp under AddressSanitizer + UBSan, driven by a C test program."""
    gpp = shutil.which("g++")
    if gpp is None:
        pytest.skip("no g++")
    src = os.path.join(ROOT, "lm_head_linear_amd", "csrc", "flce_check.cpp")
    drv = os.path.join(ROOT, "tests", "csrc", "check_driver.cpp")
    exe = str(tmp_path / "check_driver")
    r = subprocess.run([gpp, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
                        src, drv, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def build_c_caller(out_dir) -> str:
    """tests/csrc/c_caller.c compiled as C99 (warnings are errors) and linked
    against the library and the HIP runtime; returns the executable's path."""
    from lm_head_linear_amd import _lib
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    libdir = os.path.dirname(_lib.LIB_PATH)
    exe = os.path.join(str(out_dir), "c_caller")
    r = subprocess.run([gcc, "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "csrc", "c_caller.c"), "-o", exe,
                        "-L", libdir, "-lflce", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                        "-lm", f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return exe


def test_header_and_library_usable_from_c(lib, tmp_path):
    """The boundary is plain C: the header compiles as C99 and a C program
    links against the library (it runs in the GPU tests)."""
    assert os.path.exists(build_c_caller(tmp_path))


# ------------------------------------------------------- forward-only entry
def _fargs(**kw):
    a = dict(zip(("h", "W", "labels", "N", "H", "V", "ignore", "softcap", "red", "T", "loss",
                  "nt", "dH", "dW", "stream", "dtype", "mb", "acc", "ws", "wsb", "status",
                  "lse"), _args(**kw)))
    return [a[k] for k in ("h", "W", "labels", "N", "H", "V", "ignore", "softcap", "red", "T",
                           "loss", "nt", "stream", "dtype", "mb", "ws", "wsb", "status", "lse")]


def test_forward_workspace_is_the_forward_part(lib):
    """The forward-only plan carves the log-sum-exp partials and per-token
    arrays (and, for bf16, the gathered tokens: positions, labels, hidden
    rows) but no gradient chunk and no dH accumulator."""
    for N, H, V in [(8192, 4096, 131072), (8192, 3584, 256000), (32, 64, 1024), (1, 8, 1)]:
        for dt in (0, 1):
            f = lib.flce_forward_workspace_size(N, H, V, dt)
            full = lib.flce_workspace_size(N, H, V, dt)
            assert 0 < f < full
            n_tiles = -(-V // (256 if dt == 1 else 64))
            gather = (N * H * 2 + 12 * N + 4 * (N // 1024 + 1) + 4 * 256) if dt == 1 else 0
            assert f <= 256 + n_tiles * (N + 256) * 8 + 3 * (N + 256) * 8 + 4 * 256 + gather
    assert lib.flce_forward_workspace_size(-1, 8, 8, 1) == 0
    assert lib.flce_forward_workspace_size(0, 8, 8, 1) > 0


def test_forward_check_args_ok(lib):
    assert lib.flce_forward_check_args(*_fargs()) == 0
    assert lib.flce_forward_check_args(*_fargs(dtype=0, H=3)) == 0
    # a workspace big enough for the forward only is accepted by the forward entry
    f = lib.flce_forward_workspace_size(64, 64, 128, 1)
    assert lib.flce_forward_check_args(*_fargs(wsb=f)) == 0
    assert lib.flce_check_args(*_args(wsb=f)) == 3
    assert lib.flce_forward_check_args(*_fargs(wsb=f - 1)) == 3


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 1), (dict(H=0), 1), (dict(V=0), 1),
    (dict(red=2), 1), (dict(dtype=5), 1),
    (dict(softcap=-1.0), 1), (dict(softcap=float("nan")), 1), (dict(mb=float("inf")), 1),
    (dict(red=1, T=10), 1),
    (dict(h=None), 1), (dict(W=None), 1), (dict(labels=None), 1), (dict(loss=None), 1),
    (dict(nt=None), 1),
    (dict(h=A16 + 8), 2), (dict(W=A16 * 64 + 4), 2),
    (dict(ws=None), 3), (dict(ws=A16 * 1024 + 128), 3), (dict(wsb=16), 3),
])
def test_forward_check_args_errors(lib, kw, code):
    assert lib.flce_forward_check_args(*_fargs(**kw)) == code


def test_forward_rejects_before_launch(lib):
    assert lib.flce_forward(*_fargs(N=-1)) == 1
    assert lib.flce_forward(*_fargs(wsb=1)) == 3
    assert lib.flce_forward_check_args(*_fargs(N=0, h=None, labels=None)) == 0


def test_python_forward_validation_without_gpu():
    import lm_head_linear_amd as m
    h = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        m.flce_forward(h, W, y)                   # CPU tensors: refused, no fallback
    with torch.no_grad(), pytest.raises(ValueError):
        m.fused_linear_cross_entropy(h, y, W)     # forward-only route, same refusal


# ------------------------------------------------- logits-returning forward
LG = 1 << 42          # fake logits address past every other fake buffer


def _largs(logits=LG, ld=None, ldt=0, **kw):
    a = _fargs(**kw)
    V = kw.get("V", 128)
    return a + [logits, V if ld is None else ld, ldt]


def test_forward_logits_check_args_ok(lib):
    assert lib.flce_forward_logits_check_args(*_largs()) == 0
    assert lib.flce_forward_logits_check_args(*_largs(ldt=1, ld=129)) == 0   # any ld >= V
    assert lib.flce_forward_logits_check_args(*_largs(dtype=0, H=3, ld=1000)) == 0
    # the forward-only entry's workspace is enough (this entry does not gather
    # the tokens, so it needs less); too little is refused
    f = lib.flce_forward_workspace_size(64, 64, 128, 1)
    assert lib.flce_forward_logits_check_args(*_largs(wsb=f)) == 0
    assert lib.flce_forward_logits_check_args(*_largs(wsb=1024)) == 3
    # N = 0: no logits buffer needed
    assert lib.flce_forward_logits_check_args(*_largs(N=0, h=None, labels=None, logits=None)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), 1), (dict(ld=127), 1), (dict(ld=(1 << 31) + 1), 1), (dict(ldt=2), 1),
    (dict(logits=A16), 1),                 # overlaps h
    (dict(logits=A16 * 64 - 64 * 128 * 4 + 4), 1),   # last row runs into W
    (dict(logits=A16 * 128 + 8), 1),       # overlaps labels
    (dict(logits=A16 * 129), 1),           # overlaps loss
    (dict(logits=A16 * 1024 + 4096), 1),   # inside the workspace
    (dict(logits=LG + 2), 2),              # float32 logits not 4-byte aligned
    (dict(logits=LG + 1, ldt=1), 2),       # bf16 logits not 2-byte aligned
    (dict(N=-1), 1), (dict(wsb=16), 3),
])
def test_forward_logits_check_args_errors(lib, kw, code):
    assert lib.flce_forward_logits_check_args(*_largs(**kw)) == code


def test_forward_logits_rejects_before_launch(lib):
    assert lib.flce_forward_logits(*_largs(N=-1)) == 1
    assert lib.flce_forward_logits(*_largs(wsb=1)) == 3
    assert lib.flce_forward_logits(*_largs(ld=3)) == 1


def test_forward_logits_ordering_of_errors(lib):
    """Argument errors (an overlapping logits buffer) are reported before an
    unsupported layout, which is reported before the workspace."""
    assert lib.flce_forward_logits_check_args(*_largs(H=12, logits=A16)) == 1
    assert lib.flce_forward_logits_check_args(*_largs(wsb=16, logits=LG + 2)) == 2


def test_python_forward_logits_validation_without_gpu():
    import lm_head_linear_amd as m
    h = torch.zeros(4, 8, dtype=torch.bfloat16)
    W = torch.zeros(16, 8, dtype=torch.bfloat16)
    y = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        m.flce_forward_logits(h, W, y)            # CPU tensors: refused, no fallback


# ------------------------------------------- float32 gradients for bf16 inputs
def test_f32grad_plan(lib):
    """G kept as a hi + lo pair: half the vocabulary rows per chunk, no dH
    accumulator (dH is float32 itself), still within N*V*4/8."""
    for N, H, V in [(8192, 4096, 131072), (8192, 3584, 256000), (16384, 4096, 131072)]:
        assert lib.flce_vocab_chunk_ex(N, H, V, 1, 0) <= lib.flce_vocab_chunk(N, H, V, 1) // 2 + 256
        ws = lib.flce_workspace_size_ex(N, H, V, 1, 0)
        assert 0 < ws <= N * V * 4 // 8
    # same-dtype calls are exactly the plain entry points
    assert lib.flce_workspace_size_ex(8192, 4096, 131072, 1, 1) == lib.flce_workspace_size(8192, 4096, 131072, 1)
    assert lib.flce_workspace_size_ex(32, 64, 1024, 0, 0) == lib.flce_workspace_size(32, 64, 1024, 0)
    assert lib.flce_workspace_size_ex(32, 64, 1024, 0, 1) == 0      # f32 inputs, bf16 grads
    assert lib.flce_workspace_size_ex(32, 64, 1024, 1, 7) == 0


@pytest.mark.parametrize("kw,grad,code", [
    (dict(), 0, 0), (dict(), 1, 0),
    (dict(dtype=0, H=3), 0, 0),
    (dict(dtype=0), 1, 2),                  # float32 inputs with bf16 gradients
    (dict(), 5, 1),                         # unknown gradient dtype
    (dict(dW=A16 * 512 + 4), 0, 2),         # float32 gradients still need 16-byte alignment
    (dict(dH=A16 * 512), 0, 1),             # dH overlapping dW
    (dict(wsb=16), 0, 3),
])
def test_check_args_ex(lib, kw, grad, code):
    assert lib.flce_check_args_ex(*_args(**kw), grad) == code


def test_f32grad_workspace_check(lib):
    need = lib.flce_workspace_size_ex(64, 64, 128, 1, 0)
    assert lib.flce_check_args_ex(*_args(wsb=need), 0) == 0
    assert lib.flce_check_args_ex(*_args(wsb=need - 1), 0) == 3
    assert lib.flce_forward_backward_ex(*_args(wsb=1), 0) == 3      # rejected before launch


# ------------------------------------------------------ no-recompute variant
def _dh_segments(M, H, K):
    """The split-K rule of the dH GEMM restated: with fewer than 128 output tiles
    of 256 x 256, up to 4 segments (one per CU share), each of at least 2048 k,
    rounded to a multiple of 64; 1 when not split."""
    tiles = -(-M // 256) * -(-H // 256)
    s = min(256 // tiles, 4, K // 2048)
    if tiles >= 128 or s < 2:
        return 1
    kseg = -(-K // s)
    kseg = -(-kseg // 64) * 64
    return -(-K // kseg)


def test_dh_split_workspace(lib):
    """The recompute path carves segs x N x H float32 partials exactly when dH
    has few output tiles: the small configuration (32 tiles) splits its
    32000-row vocabulary into 4 segments, the large-vocab one (512 tiles) does
    not split."""
    small = lib.flce_workspace_size(2048, 1024, 32000, 1)
    assert _dh_segments(2048, 1024, 32000) == 4
    assert small >= 4 * 2048 * 1024 * 4 + 32000 * 2048 * 2
    assert _dh_segments(8192, 4096, 16384) == 1
    big = lib.flce_workspace_size(8192, 4096, 131072, 1)
    # G chunk + float32 dH running sum + the gathered rows of the kept tokens
    assert big < 16384 * 8192 * 2 + 8192 * 4096 * 4 + 8192 * 4096 * 2 + (64 << 20)


def test_nr_plan(lib):
    # default chunk: min(N, 8192) rounded up to the tile
    assert lib.flce_token_chunk_nr(8192, 4096, 131072, 1, 0) == 8192
    assert lib.flce_token_chunk_nr(16384, 4096, 131072, 1, 0) == 8192
    assert lib.flce_token_chunk_nr(600, 64, 1000, 1, 0) == 768
    assert lib.flce_token_chunk_nr(8192, 4096, 131072, 1, 1000) == 1024
    assert lib.flce_token_chunk_nr(8192, 4096, 131072, 1, 100000) == 8192
    # the chunk's probabilities dominate the workspace: nc x roundup(V, 256) x 2 bytes,
    # plus the float32 partial products of a split-K dH when its output has few tiles,
    # plus, with several token chunks, the float32 [V][H] running sum of dW, plus the
    # gathered tokens (their rows, positions and labels)
    for N, H, V, tc in [(8192, 4096, 131072, 0), (8192, 3584, 256000, 2048), (600, 64, 1000, 256),
                        (16384, 4096, 131072, 512), (16384, 4096, 131072, 0)]:
        nc = lib.flce_token_chunk_nr(N, H, V, 1, tc)
        ws = lib.flce_workspace_size_nr(N, H, V, 1, tc)
        vp = -(-V // 256) * 256
        segs = _dh_segments(nc, H, V)
        split = segs * nc * H * 4 if segs > 1 else 0
        acc = V * H * 4 if nc < N else 0
        gather = N * H * 2                        # the gathered hidden rows
        lo = nc * vp * 2 + split + acc + gather
        assert lo <= ws <= lo + (vp // 256) * nc * 8 + 4 * nc * 4 + 8 * N + 12 * N + 8192
    assert lib.flce_workspace_size_nr(64, 64, 128, 0, 0) == 0        # float32: not offered
    assert lib.flce_workspace_size_nr(-1, 64, 128, 1, 0) == 0


@pytest.mark.parametrize("kw,tc,code", [
    (dict(), 0, 0), (dict(), 256, 0),
    (dict(dtype=0), 0, 2),            # float32 inputs
    (dict(), -5, 2),
    (dict(red=1, T=7), 0, 1), (dict(dH=None), 0, 1), (dict(H=12), 0, 0),
    (dict(wsb=16), 0, 3), (dict(ws=A16 * 1024 + 64), 0, 3),
])
def test_check_args_nr(lib, kw, tc, code):
    assert lib.flce_check_args_nr(*_args(**kw), tc) == code


def test_nr_workspace_and_rejection(lib):
    need = lib.flce_workspace_size_nr(64, 64, 128, 1, 0)
    assert lib.flce_check_args_nr(*_args(wsb=need), 0) == 0
    assert lib.flce_check_args_nr(*_args(wsb=need - 1), 0) == 3
    assert lib.flce_forward_backward_nr(*_args(wsb=1), 0) == 3       # before any launch


def test_shapes_beyond_the_index_range_are_refused(lib):
    """The bf16 kernels address tiles with 32-bit offsets: a hidden size (row
    length of h and W) above 2^22 elements, or a no-recompute probability row
    above 2^22, is refused as unsupported instead of wrapping."""
    big = dict(N=1, V=1)            # keep the fake buffers far apart
    assert lib.flce_check_args(*_args(H=(1 << 22) + 8, **big)) == 2
    assert lib.flce_check_args(*_args(H=1 << 22, **big)) == 0
    assert lib.flce_check_args(*_args(dtype=0, H=(1 << 22) + 8, **big)) == 0   # float32 path
    assert lib.flce_workspace_size_nr(64, 64, (1 << 22) + 1, 1, 0) == 0
    assert lib.flce_check_args_nr(*_args(V=(1 << 22) + 1, H=8), 0) == 2
    assert lib.flce_check_args_nr(*_args(V=1 << 22, H=8), 0) == 0
    # small batches with a huge vocabulary stay supported (G chunk rows are short)
    assert lib.flce_check_args(*_args(N=8, V=1 << 23, H=8)) == 0


def test_noalloc_refusals_before_any_launch(lib):
    """flce_forward_noalloc refuses a problem whose forward workspace exceeds
    its fixed scratch, and bad arguments, before touching the GPU."""
    from lm_head_linear_amd import _lib
    N, H, V = 16384, 64, 1 << 20

    def scratch(N, V):          # the ungathered forward: partials and per-token arrays
        npad = -(-N // 256) * 256
        return -(-V // 256) * npad * 8 + 16 * npad + 4096
    assert scratch(N, V) > _lib.NOALLOC_SCRATCH_BYTES
    for n, v in ((16384, 131072), (8192, 256000), (8192, 131072), (2048, 32000)):
        assert scratch(n, v) <= _lib.NOALLOC_SCRATCH_BYTES, (n, v)

    def call(**kw):
        a = dict(h=A16, W=A16 * 64, labels=A16 * 128, N=N, H=H, V=V, ignore=-100, softcap=0.0,
                 red=0, T=0, loss=A16 * 129, nt=A16 * 130, stream=None, dtype=1, mb=1.0,
                 status=None, lse=None)
        a.update(kw)
        return lib.flce_forward_noalloc(*[a[k] for k in ("h", "W", "labels", "N", "H", "V",
                                                         "ignore", "softcap", "red", "T", "loss",
                                                         "nt", "stream", "dtype", "mb", "status",
                                                         "lse")])
    assert call() == _lib.ERR_SCRATCH
    assert call(mb=-1.0) == _lib.ERR_ARG
    assert call(H=12) == _lib.ERR_SCRATCH          # padded copies count against it
    assert call(loss=None) == _lib.ERR_ARG


def test_noalloc_scratch_size_matches_header():
    from lm_head_linear_amd import _lib
    src = open(HEADER).read()
    m = re.search(r"#define FLCE_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", src)
    assert m, "FLCE_NOALLOC_SCRATCH_BYTES"
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES
