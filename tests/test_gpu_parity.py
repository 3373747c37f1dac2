"""GPU parity: the HIP path (through the C-ABI) against the float64 oracle on
identical seeded inputs, element by element, at sizes the oracle finishes in
seconds -- several tiles, ragged tails in tokens, hidden size and vocabulary,
several backward chunks -- plus the edge cases of the method."""
import math
import os

import numpy as np
import pytest
import torch

import flce_inputs as fi
from oracle import flce_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_linear_amd._lib as L
    L.load()          # fails loudly when libflce.so is missing
    yield


@pytest.fixture
def vchunk(monkeypatch):
    def set_chunk(v):
        monkeypatch.setenv("FLCE_VCHUNK", str(v))
    return set_chunk


# ------------------------------------------------------------ the configurations
def test_config1_tiny_fp32():
    w = fi.make_workload(1)
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    assert r.num_tokens == 29
    gu.assert_parity(w, g, r)


def test_config2_small_bf16():
    w = fi.make_workload(2)
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    assert r.num_tokens == 1946
    gu.assert_parity(w, g, r)


# ------------------------------------------------------------ ragged, multi-tile, multi-chunk
@pytest.mark.parametrize("N,H,V,chunk", [
    (600, 264, 1500, 512),      # ragged tokens, K tail, ragged vocab, 3 chunks
    (257, 64, 257, 0),          # one past a tile in tokens and vocab
    (1, 8, 2, 0),               # smallest bf16 shape
    (1000, 512, 3000, 1024),    # 3 chunks, ragged last chunk
    (513, 136, 777, 256),       # many small chunks
])
def test_ragged_bf16(N, H, V, chunk, vchunk):
    if chunk:
        vchunk(chunk)
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + V, ignore_frac=0.1)
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    gu.assert_parity(w, g, r)


@pytest.mark.parametrize("N,H,V,chunk", [(130, 70, 301, 128), (64, 64, 64, 0), (3, 5, 7, 0)])
def test_ragged_fp32(N, H, V, chunk, vchunk):
    if chunk:
        vchunk(chunk)
    w = fi.make_custom(N, H, V, dtype=torch.float32, seed=N + V, ignore_frac=0.2)
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    gu.assert_parity(w, g, r)


# ------------------------------------------------------------ options
@pytest.mark.parametrize("s", [30.0, 2.0])
def test_softcap_bf16(s, vchunk):
    vchunk(512)
    w = fi.make_custom(700, 256, 1200, dtype=torch.bfloat16, seed=11, w_std=0.03 if s > 10 else 0.3,
                       softcap=s)
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    gu.assert_parity(w, g, r)


def test_softcap_fp32():
    w = fi.make_custom(90, 48, 200, dtype=torch.float32, seed=12, w_std=0.5, softcap=1.5)
    gu.assert_parity(w, gu.run_gpu(w), gu.run_oracle(w))


def test_mean_zipf_prefix_mask():
    """Config-3 recipe at a small size: Zipf labels, first quarter masked, 'mean'."""
    w = fi.make_custom(1024, 256, 4096, dtype=torch.bfloat16, seed=13, labels="zipf",
                       ignore_frac=0.0, reduction="mean")
    w.labels[:, :256] = fi.IGNORE_INDEX
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    assert g["num_tokens"] == 0 and r.num_tokens == 0
    gu.assert_parity(w, g, r)


@pytest.mark.parametrize("T", [1000, 2500])
def test_sum_with_external_count(T):
    w = fi.make_custom(1100, 128, 2000, dtype=torch.bfloat16, seed=14, num_label_tokens=T)
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    assert g["num_tokens"] == r.num_tokens == w.expected_valid
    gu.assert_parity(w, g, r)


def test_mb_scale():
    w = fi.make_custom(300, 64, 500, dtype=torch.bfloat16, seed=15, reduction="mean")
    s = float(np.float32(0.375))
    gu.assert_parity(w, gu.run_gpu(w, mb_scale=s), gu.run_oracle(w, mb_scale=s))


@pytest.mark.parametrize("path", ["recompute", "f32grad", "norecompute", "fp32"])
@pytest.mark.parametrize("s", [0.0, 1e-3, 0.375])
def test_mb_scale_every_path(path, s, vchunk):
    """The micro-batch scale (twinkle PR 335, "PR information", item 2) on every
    gradient path, including 0 (loss 0, zero gradients, no NaN) and a small
    scale, against the oracle with the same scale, with and without a softcap
    and over several backward chunks."""
    vchunk(256)
    dt = torch.float32 if path == "fp32" else torch.bfloat16
    for cap in (0.0, 2.0):
        w = fi.make_custom(300, 64, 700, dtype=dt, seed=16, w_std=0.3, softcap=cap,
                           reduction="sum", ignore_frac=0.1)
        kw = {}
        if path == "f32grad":
            kw["grad_dtype"] = torch.float32
        elif path == "norecompute":
            kw.update(recompute=False, token_chunk=256)
        g = gu.run_gpu(w, mb_scale=float(np.float32(s)), **kw)
        r = gu.run_oracle(w, mb_scale=float(np.float32(s)))
        if path == "f32grad":
            # float32 gradients: the float32 tolerance
            assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
            gu.assert_loss(g["loss"], r.loss64)
            gu.assert_grad("dH", g["dH"], r.dH, gu.GRAD_TOL[torch.float32])
            gu.assert_grad("dW", g["dW"], r.dW, gu.GRAD_TOL[torch.float32])
        else:
            gu.assert_parity(w, g, r)
        if s == 0.0:
            assert g["loss"] == 0.0
            assert bool((g["dH"] == 0).all()) and bool((g["dW"] == 0).all())


def test_negative_mb_scale_refused():
    """A negative micro-batch scale is an argument error on every entry point:
    nothing is launched and the outputs keep their contents."""
    import lm_head_linear_amd as m
    w = fi.make_custom(64, 64, 300, dtype=torch.bfloat16, seed=17)
    dev = gu.device()
    h, W = w.h.reshape(-1, w.H).to(dev), w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    loss = torch.full((), 7.0, device=dev)
    dW = torch.full_like(W, 3.0)
    for kw in ({}, {"grad_dtype": torch.float32}, {"recompute": False}):
        dWk = dW if not kw.get("grad_dtype") else torch.full(W.shape, 3.0, device=dev)
        with pytest.raises(m.FlceError) as e:
            m.flce_forward_backward(h, W, y, mb_scale=-0.5, loss=loss, dW=dWk, **kw)
        assert e.value.code == 1
    with pytest.raises(m.FlceError):
        m.flce_forward(h, W, y, mb_scale=-0.5, loss=loss)
    torch.cuda.synchronize()
    assert loss.item() == 7.0 and bool((dW == 3.0).all())


def test_ignore_index_inside_vocab():
    w = fi.make_custom(400, 64, 300, dtype=torch.bfloat16, seed=16, ignore_frac=0.0,
                       ignore_index=5)
    w.labels[0, ::3] = 5
    g = gu.run_gpu(w)
    r = gu.run_oracle(w)
    gu.assert_parity(w, g, r)


# ------------------------------------------------------------ edge cases
@pytest.mark.parametrize("reduction", ["sum", "mean"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_all_ignored_gives_exact_zero(reduction, dtype):
    w = fi.make_custom(300, 64, 700, dtype=dtype, seed=17, ignore_frac=1.0, reduction=reduction)
    assert bool((w.labels == fi.IGNORE_INDEX).all())
    g = gu.run_gpu(w)
    assert g["loss"] == 0.0 and not math.isnan(g["loss"])
    assert g["num_tokens"] == 0
    assert bool((g["dH"] == 0).all()) and bool((g["dW"] == 0).all())


def test_pages_example_after_roll():
    """[-100, 3, -100, -100] rolled and causally shifted leaves no target: 0, not NaN."""
    dev = gu.device()
    lab = torch.roll(torch.tensor([-100, 3, -100, -100]), -1)[1:]
    w = fi.make_custom(3, 16, 50, dtype=torch.bfloat16, seed=18, ignore_frac=0.0)
    w.labels = lab.view(1, 3).clone()
    for red in ("sum", "mean"):
        w.reduction = red
        g = gu.run_gpu(w)
        assert g["loss"] == 0.0 and g["num_tokens"] == 0
        assert bool((g["dH"] == 0).all()) and bool((g["dW"] == 0).all())
    del dev


@pytest.mark.parametrize("accumulate", [False, True])
def test_empty_batch(accumulate):
    import lm_head_linear_amd as m
    dev = gu.device()
    W = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    dW = torch.full_like(W, 7.0)
    loss, nt, dH, dW = m.flce_forward_backward(h, W, y, dW=dW, accumulate_dW=accumulate)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nt.item() == 0 and dH.shape == (0, 64)
    assert bool((dW == (7.0 if accumulate else 0.0)).all())


def test_invalid_label_fails_closed():
    w = fi.make_custom(200, 64, 300, dtype=torch.bfloat16, seed=19)
    w.labels[0, 7] = 300            # out of range
    g = gu.run_gpu(w)
    assert g["status"] == 5
    assert math.isnan(g["loss"])
    assert bool(torch.isnan(g["dH"][7].float()).all())
    w.labels[0, 7] = -3
    g = gu.run_gpu(w)
    assert g["status"] == 5 and math.isnan(g["loss"])
    with pytest.raises(ValueError):
        gu.run_oracle(w)


def test_vocab_one_and_two():
    w = fi.make_custom(100, 16, 1, dtype=torch.bfloat16, seed=20)
    g = gu.run_gpu(w)
    assert g["loss"] == 0.0
    assert bool((g["dH"] == 0).all()) and bool((g["dW"] == 0).all())
    w2 = fi.make_custom(100, 16, 2, dtype=torch.bfloat16, seed=21, w_std=0.5)
    gu.assert_parity(w2, gu.run_gpu(w2), gu.run_oracle(w2))


def test_zero_weight_gives_log_v():
    w = fi.make_custom(333, 64, 1024, dtype=torch.bfloat16, seed=22)
    w.W.zero_()
    g = gu.run_gpu(w)
    n = w.expected_valid
    assert abs(g["loss"] - n * 10 * math.log(2.0)) <= 1e-5 * n * 10 * math.log(2.0)
    assert bool((g["dH"] == 0).all())


# ------------------------------------------------------------ determinism, micro-batches
def test_bitwise_deterministic(vchunk):
    vchunk(512)
    w = fi.make_custom(700, 128, 1500, dtype=torch.bfloat16, seed=23)
    a = gu.run_gpu(w)
    b = gu.run_gpu(w)
    assert a["loss"] == b["loss"]
    assert torch.equal(a["dH"], b["dH"]) and torch.equal(a["dW"], b["dW"])
    assert torch.equal(a["lse"], b["lse"])


def test_micro_batches_accumulate_dW():
    """Four micro-batches with a shared external count and accumulate_dW add up to
    one call over the whole batch (config-5 recipe, small size)."""
    import lm_head_linear_amd as m
    dev = gu.device()
    N, H, V = 1024, 128, 2048
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=24, ignore_frac=0.0)
    w.labels[0, 300:420] = fi.IGNORE_INDEX
    T = int((w.labels != fi.IGNORE_INDEX).sum())
    w.num_label_tokens = T
    r = gu.run_oracle(w)
    h = w.h.reshape(-1, H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    dW = torch.empty_like(W)
    dH = torch.empty_like(h)
    total = 0.0
    ntok = 0
    for k in range(4):
        s = slice(256 * k, 256 * (k + 1))
        loss, nt, _, _ = m.flce_forward_backward(h[s], W, y[s], num_label_tokens=T,
                                                 dH=dH[s], dW=dW, accumulate_dW=k > 0)
        total += loss.item()
        ntok += nt.item()
    torch.cuda.synchronize()
    assert ntok == T == r.n_valid
    gu.assert_loss(total, r.loss64)
    gu.assert_grad("dH", dH, r.dH, 2e-2)
    gu.assert_grad("dW", dW, r.dW, 2e-2)
    assert bool((dH[300:420] == 0).all())


# ------------------------------------------------------------ Python module / autograd
def test_module_and_autograd():
    import lm_head_linear_amd as m
    dev = gu.device()
    w = fi.make_custom(256, 64, 512, dtype=torch.bfloat16, seed=25, reduction="mean")
    r = gu.run_oracle(w)
    h = w.h.to(dev).requires_grad_(True)
    W = w.W.to(dev).requires_grad_(True)
    mod = m.FusedLinearCrossEntropy(reduction="mean")
    loss = mod(h, w.labels.to(dev), W)
    assert loss.dtype == torch.float32
    (2.0 * loss).backward()
    assert int(mod.num_tokens.item()) == 0
    gu.assert_loss(loss.item(), r.loss64)
    gu.assert_grad("dH", h.grad.reshape(-1, 64), 2.0 * r.dH, 2e-2)
    gu.assert_grad("dW", W.grad, 2.0 * r.dW, 2e-2)
