"""The forward keeps the probabilities of the first vocabulary chunks (when dW
is overwritten, all but the last of them in the rows of dW the backward has
not yet written, the last in the workspace), whose G is then formed in place
instead of recomputing their logits. GPU parity against the oracle for shapes
that keep 4 of 16 chunks, 4 of 6 (softcap, 'mean') and all 4 (the short last
chunk in the workspace), with dW filled with NaN before the call (every row
must be overwritten) and a second call giving the same bits; with
accumulate_dW only chunk 0 is kept and the gradient is added to the dW
already there."""
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


@pytest.fixture
def vchunk(monkeypatch):
    def set_chunk(v):
        monkeypatch.setenv("FLCE_VCHUNK", str(v))
    return set_chunk


@pytest.mark.parametrize("N,H,V,chunk,cap,red,kept", [
    (300, 512, 4000, 256, 0.0, "sum", 4),      # 16 chunks, 4 kept
    (600, 1024, 3000, 512, 30.0, "mean", 4),   # 6 chunks, 4 kept, softcap
    (100, 768, 900, 256, 0.0, "sum", 4),       # 4 chunks, all kept (the short last one too)
])
def test_kept_chunks_parity(N, H, V, chunk, cap, red, kept, vchunk):
    import lm_head_linear_amd as m
    vchunk(chunk)
    assert m.flce_kept_chunks(N, H, V, torch.bfloat16) == kept
    assert m.flce_kept_chunks(N, H, V, torch.bfloat16, True) == 1
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + H, softcap=cap, reduction=red)
    dev = gu.device()
    dW = torch.full((V, H), float("nan"), dtype=torch.bfloat16, device=dev)
    g = gu.run_gpu(w, dW=dW)
    r = gu.run_oracle(w)
    gu.assert_parity(w, g, r)
    again = gu.run_gpu(w)
    assert again["loss"] == g["loss"]
    assert torch.equal(again["dW"], g["dW"]) and torch.equal(again["dH"], g["dH"])


def test_kept_chunks_not_used_when_dW_is_added_to(vchunk):
    vchunk(256)
    N, H, V = 300, 512, 4000
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=31)
    r = gu.run_oracle(w)
    scale = float(np.abs(r.dW).max())
    base = (torch.randn(V, H, generator=torch.Generator().manual_seed(5)) * scale).to(torch.bfloat16)
    dW = base.to(gu.device())
    g = gu.run_gpu(w, dW=dW, accumulate_dW=True)
    assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
    gu.assert_loss(g["loss"], r.loss64)
    gu.assert_grad("dH", g["dH"], r.dH, 2e-2)
    gu.assert_grad("dW", g["dW"], base.double().numpy() + r.dW, 2e-2)


def test_kept_chunks_with_gradients_16_byte_aligned_only(vchunk):
    """dW and dH only 16-byte aligned (the ABI's requirement), so the kept
    chunks' G in dW starts off a cache line: the same values as with aligned
    buffers."""
    vchunk(256)
    N, H, V = 300, 512, 4000
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=32)
    dev = gu.device()
    big_w = torch.full((V * H + 64,), float("nan"), dtype=torch.bfloat16, device=dev)
    big_h = torch.full((N * H + 64,), float("nan"), dtype=torch.bfloat16, device=dev)
    dW = big_w[8:8 + V * H].view(V, H)             # 16 bytes past a 256-byte boundary
    dH = big_h[24:24 + N * H].view(N, H)           # 48 bytes past
    assert dW.data_ptr() % 256 == 16 and dH.data_ptr() % 256 == 48
    g = gu.run_gpu(w, dW=dW, dH=dH)
    ref = gu.run_gpu(w)
    assert g["status"] == 0 and g["loss"] == ref["loss"]
    assert torch.equal(g["dW"], ref["dW"]) and torch.equal(g["dH"], ref["dH"])
    gu.assert_parity(w, g, gu.run_oracle(w))
