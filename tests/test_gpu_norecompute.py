"""GPU parity of the no-recompute variant (flce_forward_backward_nr): loss,
count, lse, dH and dW against the float64 oracle at the bf16 tolerances on
identical seeded inputs, over one and several token chunks (dW added up over
the chunks), with the softcap, both reductions, an external count and the
micro-batch scale, plus the edge cases; and agreement with the recompute
path."""
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


def _check(w, token_chunk=0, **kw):
    g = gu.run_gpu(w, recompute=False, token_chunk=token_chunk, **kw)
    r = gu.run_oracle(w, **{k: v for k, v in kw.items() if k in ("mb_scale", "num_label_tokens")})
    gu.assert_parity(w, g, r)
    return g, r


def test_config2_small():
    w = fi.make_workload(2)
    g, r = _check(w)
    c, _ = _check(w, token_chunk=512)          # 4 token chunks
    # the recompute path agrees closely (differently rounded partial sums)
    b = gu.run_gpu(w)
    assert abs(g["loss"] - b["loss"]) <= 1e-6 * abs(b["loss"])
    assert float((g["lse"] - b["lse"]).abs().max()) <= 1e-5 * float(b["lse"].abs().max())


@pytest.mark.parametrize("N,H,V,tc", [
    (600, 264, 1500, 256),      # 3 token chunks, ragged tokens, K tail, ragged vocab
    (257, 64, 257, 0),          # one chunk, one past a tile
    (1, 8, 2, 0),
    (1000, 512, 3000, 256),     # 4 chunks, the last one short
    (513, 136, 777, 512),
])
def test_ragged(N, H, V, tc):
    _check(fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=200 + N), token_chunk=tc)


@pytest.mark.parametrize("s", [30.0, 2.0])
def test_softcap(s):
    w = fi.make_custom(700, 136, 1000, dtype=torch.bfloat16, seed=201, w_std=0.5)
    w.softcap = s
    _check(w, token_chunk=256)


def test_mean_zipf_scale_and_external_count():
    w = fi.make_custom(900, 128, 1500, dtype=torch.bfloat16, seed=202, labels="zipf")
    w.reduction = "mean"
    _check(w, token_chunk=256, mb_scale=0.75)
    w.reduction = "sum"
    w.num_label_tokens = 2000
    g, _ = _check(w, token_chunk=512)
    assert g["num_tokens"] == w.expected_valid


def test_ignore_index_inside_vocab():
    w = fi.make_custom(400, 64, 300, dtype=torch.bfloat16, seed=203, ignore_index=5)
    _check(w, token_chunk=256)


def test_accumulate_dW_over_calls():
    """Two calls over halves of the batch with accumulate_dW: the oracle's single call."""
    import lm_head_linear_amd as m
    w = fi.make_custom(1024, 128, 2000, dtype=torch.bfloat16, seed=204)
    w.num_label_tokens = w.expected_valid
    r = gu.run_oracle(w)
    dev = gu.device()
    h = w.h.reshape(-1, w.H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    dH = torch.empty_like(h)
    dW = torch.empty_like(W)
    total = 0.0
    for i in range(2):
        s = slice(i * 512, (i + 1) * 512)
        loss, _, _, _ = m.flce_forward_backward(h[s], W, y[s], num_label_tokens=w.num_label_tokens,
                                                dH=dH[s], dW=dW, accumulate_dW=i > 0,
                                                recompute=False, token_chunk=256)
        total += loss.item()
    torch.cuda.synchronize()
    gu.assert_loss(total, r.loss64)
    gu.assert_grad("dH", dH, r.dH, 2e-2)
    gu.assert_grad("dW", dW, r.dW, 2e-2)


@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_all_ignored_exact_zero(reduction):
    w = fi.make_custom(600, 64, 500, dtype=torch.bfloat16, seed=205)
    w.labels.fill_(w.ignore_index)
    w.reduction = reduction
    g = gu.run_gpu(w, recompute=False, token_chunk=256)
    assert g["loss"] == 0.0 and g["num_tokens"] == 0
    assert bool((g["dH"] == 0).all()) and bool((g["dW"] == 0).all())


@pytest.mark.parametrize("accumulate", [False, True])
def test_empty_batch(accumulate):
    import lm_head_linear_amd as m
    dev = gu.device()
    W = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    dW = torch.full_like(W, 7.0)
    loss, nt, dH, dW = m.flce_forward_backward(h, W, y, dW=dW, accumulate_dW=accumulate,
                                               recompute=False)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nt.item() == 0
    assert bool((dW == (7.0 if accumulate else 0.0)).all())


def test_invalid_label_fails_closed():
    w = fi.make_custom(300, 64, 300, dtype=torch.bfloat16, seed=206)
    w.labels[0, 270] = 300          # in the second token chunk
    g = gu.run_gpu(w, recompute=False, token_chunk=256)
    assert g["status"] == 5 and math.isnan(g["loss"])
    assert bool(torch.isnan(g["dH"][270].float()).all())


def test_vocab_one_and_two():
    w = fi.make_custom(300, 16, 1, dtype=torch.bfloat16, seed=207)
    g = gu.run_gpu(w, recompute=False, token_chunk=256)
    assert g["loss"] == 0.0
    assert bool((g["dH"] == 0).all()) and bool((g["dW"] == 0).all())
    _check(fi.make_custom(300, 16, 2, dtype=torch.bfloat16, seed=208, w_std=0.5), token_chunk=256)


def test_float32_inputs_refused():
    import lm_head_linear_amd as m
    dev = gu.device()
    h = torch.randn(16, 64, device=dev)
    W = torch.randn(100, 64, device=dev)
    y = torch.zeros(16, dtype=torch.int64, device=dev)
    with pytest.raises(m.FlceError):
        m.flce_forward_backward(h, W, y, recompute=False)
