"""GPU parity of the forward-only entry (flce_forward): loss, num_tokens, the
per-token lse and the status against the float64 oracle on identical seeded
inputs, and bit-identity with the forward half of flce_forward_backward (the
same kernels run on the same values), plus the edge cases of the method."""
import math

import numpy as np
import pytest
import torch

import flce_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_linear_amd._lib as L
    L.load()
    yield


def _check(w, *, mb_scale=1.0, **kw):
    f = gu.run_gpu_forward(w, mb_scale=mb_scale, **kw)
    r = gu.run_oracle(w, mb_scale=mb_scale, **kw)
    assert f["status"] == 0
    assert f["num_tokens"] == r.num_tokens
    gu.assert_loss(f["loss"], r.loss64)
    lse = gu.to_np64(f["lse"])
    assert np.abs(lse - r.lse).max() <= 1e-5 * max(1.0, np.abs(r.lse).max())
    # the forward half of the full call: identical bits
    g = gu.run_gpu(w, mb_scale=mb_scale, **kw)
    assert f["loss_t"].view(torch.int32).item() == g["loss_t"].view(torch.int32).item()
    assert f["num_tokens"] == g["num_tokens"] and f["status"] == g["status"]
    assert torch.equal(f["lse"].view(torch.int32), g["lse"].view(torch.int32))
    return f, r


def test_config1_tiny_fp32():
    _check(fi.make_workload(1))


def test_config2_small_bf16():
    _check(fi.make_workload(2))


@pytest.mark.parametrize("N,H,V", [(600, 264, 1500), (257, 64, 257), (1, 8, 2), (513, 136, 777)])
def test_ragged_bf16(N, H, V):
    _check(fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + V))


@pytest.mark.parametrize("N,H,V", [(130, 70, 301), (3, 5, 7)])
def test_ragged_fp32(N, H, V):
    _check(fi.make_custom(N, H, V, dtype=torch.float32, seed=N + V))


@pytest.mark.parametrize("s", [30.0, 2.0])
def test_softcap(s):
    w = fi.make_custom(300, 136, 1000, dtype=torch.bfloat16, seed=23, w_std=0.5)
    w.softcap = s
    _check(w)


def test_mean_and_external_count_and_scale():
    w = fi.make_custom(700, 128, 1500, dtype=torch.bfloat16, seed=24)
    w.reduction = "mean"
    f, r = _check(w, mb_scale=0.375)
    assert f["num_tokens"] == 0
    w.reduction = "sum"
    w.num_label_tokens = 2500
    f, _ = _check(w)
    assert f["num_tokens"] == w.expected_valid


@pytest.mark.parametrize("reduction", ["sum", "mean"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_all_ignored_gives_exact_zero(reduction, dtype):
    w = fi.make_custom(300, 64, 500, dtype=dtype, seed=25)
    w.labels.fill_(w.ignore_index)
    w.reduction = reduction
    f = gu.run_gpu_forward(w)
    assert f["loss"] == 0.0 and f["num_tokens"] == 0 and f["status"] == 0


def test_empty_batch():
    import lm_head_linear_amd as m
    dev = gu.device()
    W = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    loss, nt = m.flce_forward(h, W, y)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nt.item() == 0


def test_invalid_label_fails_closed():
    w = fi.make_custom(200, 64, 300, dtype=torch.bfloat16, seed=26)
    w.labels[0, 11] = 300
    f = gu.run_gpu_forward(w)
    assert f["status"] == 5 and math.isnan(f["loss"])


def test_vocab_one():
    """V = 1: lse is the single logit, so every token loss is exactly 0."""
    f, _ = _check(fi.make_custom(100, 16, 1, dtype=torch.bfloat16, seed=27))
    assert f["loss"] == 0.0


def test_module_without_grad_uses_forward_only():
    """Under torch.no_grad() the module returns the same loss bits and count as
    the training call, with no gradient attached."""
    import lm_head_linear_amd as m
    dev = gu.device()
    w = fi.make_custom(400, 128, 1000, dtype=torch.bfloat16, seed=28)
    h = w.h.to(dev)
    W = w.W.to(dev)
    y = w.labels.to(dev)
    mod = m.FusedLinearCrossEntropy(reduction="mean", logit_softcapping=5.0)
    with torch.no_grad():
        l0 = mod(h, y, W)
        n0 = int(mod.num_tokens)
    hr = h.clone().requires_grad_(True)
    l1 = mod(hr, y, W)
    assert not l0.requires_grad and l1.requires_grad
    assert n0 == int(mod.num_tokens) == 0
    assert l0.view(torch.int32).item() == l1.detach().view(torch.int32).item()
