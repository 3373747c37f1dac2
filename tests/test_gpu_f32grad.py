"""GPU parity of float32 gradients for bf16 inputs (flce_forward_backward_ex
with grad_dtype float32): dH and dW against the float64 oracle at the float32
tolerance, max |gpu - ref| <= 1e-4 * max |ref| per tensor, on identical seeded
bf16 inputs; the loss, count and lse bit-identical to the bf16-gradient call;
float32 accumulation of dW over micro-batches; and the edge cases."""
import math
import os

import numpy as np
import pytest
import torch

import flce_inputs as fi
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
TOL = gu.GRAD_TOL[torch.float32]     # 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_linear_amd._lib as L
    L.load()
    yield


@pytest.fixture
def vchunk(monkeypatch):
    def set_chunk(v):
        monkeypatch.setenv("FLCE_VCHUNK", str(v))
    return set_chunk


def _check(w, **kw):
    g = gu.run_gpu(w, grad_dtype=torch.float32, **kw)
    r = gu.run_oracle(w, **{k: v for k, v in kw.items() if k in ("mb_scale", "num_label_tokens")})
    assert g["dH"].dtype == torch.float32 and g["dW"].dtype == torch.float32
    assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
    gu.assert_loss(g["loss"], r.loss64)
    gu.assert_grad("dH", g["dH"], r.dH, TOL)
    gu.assert_grad("dW", g["dW"], r.dW, TOL)
    ign = np.flatnonzero(w.labels.reshape(-1).numpy() == w.ignore_index)
    if ign.size:
        assert bool((g["dH"][torch.from_numpy(ign).to(g["dH"].device)] == 0).all())
    # the forward part is the bf16 call's, bit for bit
    b = gu.run_gpu(w, **kw)
    assert g["loss_t"].view(torch.int32).item() == b["loss_t"].view(torch.int32).item()
    assert torch.equal(g["lse"].view(torch.int32), b["lse"].view(torch.int32))
    return g, r, b


def test_config2_small():
    w = fi.make_workload(2)
    g, r, b = _check(w)
    # float32 gradients are much closer to the oracle than bf16 ones
    e32 = np.abs(gu.to_np64(g["dW"]) - r.dW).max()
    e16 = np.abs(gu.to_np64(b["dW"]) - r.dW).max()
    assert e32 < e16 / 20, (e32, e16)


@pytest.mark.parametrize("N,H,V,chunk", [
    (600, 264, 1500, 512),      # ragged tokens, K tail, ragged vocab, 3 chunks
    (257, 64, 257, 0),
    (1, 8, 2, 0),
    (513, 136, 777, 256),       # many chunks: 2 GEMMs per part per chunk, fixed order
])
def test_ragged(N, H, V, chunk, vchunk):
    if chunk:
        vchunk(chunk)
    _check(fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=100 + N))


@pytest.mark.parametrize("s", [30.0, 2.0])
def test_softcap(s, vchunk):
    vchunk(512)
    w = fi.make_custom(300, 136, 1000, dtype=torch.bfloat16, seed=101, w_std=0.5)
    w.softcap = s
    _check(w)


def test_mean_scale_and_external_count():
    w = fi.make_custom(700, 128, 1500, dtype=torch.bfloat16, seed=102, labels="zipf")
    w.reduction = "mean"
    _check(w, mb_scale=0.625)
    w.reduction = "sum"
    w.num_label_tokens = 2000
    _check(w)


def test_micro_batches_accumulate_in_float32():
    """4 micro-batches with a shared external count, dW added up in float32:
    equal to the oracle's single call over the whole batch."""
    import lm_head_linear_amd as m
    w = fi.make_custom(1024, 128, 2000, dtype=torch.bfloat16, seed=103)
    w.num_label_tokens = w.expected_valid
    r = gu.run_oracle(w)
    dev = gu.device()
    h = w.h.reshape(-1, w.H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    dH = torch.empty(h.shape, dtype=torch.float32, device=dev)
    dW = torch.full(W.shape, 123.0, dtype=torch.float32, device=dev)   # overwritten by call 0
    total = 0.0
    for i in range(4):
        s = slice(i * 256, (i + 1) * 256)
        loss, nt, _, _ = m.flce_forward_backward(h[s], W, y[s], num_label_tokens=w.num_label_tokens,
                                                 dH=dH[s], dW=dW, accumulate_dW=i > 0,
                                                 grad_dtype=torch.float32)
        total += loss.item()
    torch.cuda.synchronize()
    gu.assert_loss(total, r.loss64)
    gu.assert_grad("dH", dH, r.dH, TOL)
    gu.assert_grad("dW", dW, r.dW, TOL)


@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_all_ignored_exact_zero(reduction):
    w = fi.make_custom(300, 64, 500, dtype=torch.bfloat16, seed=104)
    w.labels.fill_(w.ignore_index)
    w.reduction = reduction
    g = gu.run_gpu(w, grad_dtype=torch.float32)
    assert g["loss"] == 0.0 and g["num_tokens"] == 0
    assert bool((g["dH"] == 0).all()) and bool((g["dW"] == 0).all())


@pytest.mark.parametrize("accumulate", [False, True])
def test_empty_batch(accumulate):
    import lm_head_linear_amd as m
    dev = gu.device()
    W = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    dW = torch.full((300, 64), 7.0, dtype=torch.float32, device=dev)
    loss, nt, dH, dW = m.flce_forward_backward(h, W, y, dW=dW, accumulate_dW=accumulate,
                                               grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nt.item() == 0 and dH.dtype == torch.float32
    assert bool((dW == (7.0 if accumulate else 0.0)).all())


def test_invalid_label_fails_closed():
    w = fi.make_custom(200, 64, 300, dtype=torch.bfloat16, seed=105)
    w.labels[0, 9] = 300
    g = gu.run_gpu(w, grad_dtype=torch.float32)
    assert g["status"] == 5 and math.isnan(g["loss"])
    assert bool(torch.isnan(g["dH"][9]).all())


def test_float32_inputs_with_bf16_gradients_refused():
    import lm_head_linear_amd as m
    dev = gu.device()
    h = torch.randn(16, 64, device=dev)
    W = torch.randn(100, 64, device=dev)
    y = torch.zeros(16, dtype=torch.int64, device=dev)
    with pytest.raises(m.FlceError):
        m.flce_forward_backward(h, W, y, grad_dtype=torch.bfloat16)
