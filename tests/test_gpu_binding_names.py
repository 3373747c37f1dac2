"""The binding's same-named wrappers of the float32-gradient and no-recompute
entry points (flce_forward_backward_ex, flce_forward_backward_nr) give the same
bits as the keyword forms of flce_forward_backward, and match the oracle."""
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


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t.view(torch.int32) if t.dtype == torch.float32 else t   # int64 num_tokens as is


def _same(a, b):
    for x, y in zip(a, b):
        assert x.dtype == y.dtype and torch.equal(_bits(x), _bits(y))


def test_named_wrappers_equal_keyword_forms():
    import lm_head_linear_amd as m
    w = fi.make_custom(600, 72, 1300, dtype=torch.bfloat16, seed=61, ignore_frac=0.2,
                       softcap=30.0, reduction="mean")
    dev = gu.device()
    h, W, y = w.h.reshape(-1, w.H).to(dev), w.W.to(dev), w.labels.reshape(-1).to(dev)
    kw = dict(ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction)
    ex = m.flce_forward_backward_ex(h, W, y, grad_dtype=torch.float32, **kw)
    ex_kw = m.flce_forward_backward(h, W, y, grad_dtype=torch.float32, **kw)
    nr = m.flce_forward_backward_nr(h, W, y, token_chunk=256, **kw)
    nr_kw = m.flce_forward_backward(h, W, y, recompute=False, token_chunk=256, **kw)
    torch.cuda.synchronize(dev)
    _same(ex, ex_kw)
    _same(nr, nr_kw)
    r = gu.run_oracle(w)
    print("case: N=600 H=72 V=1300 softcap=30 mean", flush=True)
    for out, tol in ((ex, gu.GRAD_TOL[torch.float32]), (nr, gu.GRAD_TOL[torch.bfloat16])):
        loss, nt, dH, dW = out
        assert int(nt.item()) == r.num_tokens
        gu.assert_loss(float(loss.item()), r.loss64)
        gu.assert_grad("dH", dH, r.dH, tol)
        gu.assert_grad("dW", dW, r.dW, tol)
