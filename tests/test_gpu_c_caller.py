"""The library called from plain C (tests/csrc/c_caller.c): device memory and
copies through the HIP runtime only, no PyTorch. With W = 0 the loss, lse,
num_tokens, dH and dW have closed forms, which the program checks for a
hidden size that is a multiple of 8 and one that is not."""
import os
import subprocess

import pytest
import torch

from tests.test_abi_cpu import build_c_caller

pytestmark = pytest.mark.gpu


def test_c_caller_closed_form(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = build_c_caller(tmp_path)
    print("running", exe, flush=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c caller: all checks passed" in r.stdout
