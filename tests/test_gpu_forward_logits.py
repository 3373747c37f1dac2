"""GPU parity of the logits-returning forward (flce_forward_logits): the
stored logits against the float64 oracle's Z' element by element, within a
bound derived from float32 accumulation; the bf16 logits as the
round-to-nearest-even of the float32 ones; the loss, count, lse and status
bit-identical to flce_forward; the stored logits are the ones the lse was
formed from; nothing outside [N, V] of the caller's buffer is written."""
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
    L.load()
    yield


def _check(w, *, pad=0, mb_scale=1.0, **kw):
    V = w.W.shape[0]
    f32 = gu.run_gpu_forward_logits(w, logits_dtype=torch.float32, pad=pad, mb_scale=mb_scale,
                                    **kw)
    b16 = gu.run_gpu_forward_logits(w, logits_dtype=torch.bfloat16, pad=pad + 3,
                                    mb_scale=mb_scale, **kw)
    ref = gu.run_gpu_forward(w, mb_scale=mb_scale, **kw)
    # loss, count, lse and status: the same bits as the forward-only entry
    for o in (f32, b16):
        assert o["status"] == ref["status"] == 0
        assert o["loss_t"].view(torch.int32).item() == ref["loss_t"].view(torch.int32).item()
        assert o["num_tokens"] == ref["num_tokens"]
        assert torch.equal(o["lse"].view(torch.int32), ref["lse"].view(torch.int32))
    # float32 logits against the oracle's Z'
    h64 = w.h.reshape(-1, w.H).to(torch.float64).numpy()
    W64 = w.W.to(torch.float64).numpy()
    Z = orc.logits_rows(h64, W64, w.softcap)
    got = gu.to_np64(f32["logits"])
    err = np.abs(got - Z)
    tol = gu.logits_tolerance(w)
    worst = np.unravel_index(np.argmax(err / tol), err.shape)
    assert (err <= tol).all(), f"logit {worst}: err {err[worst]:.3e} > tol {tol[worst]:.3e}"
    print(f"logits max err {err.max():.3e}, max err/tol {(err / tol).max():.3f}")
    # the bf16 logits are the float32 ones rounded to nearest even
    assert torch.equal(b16["logits"].view(torch.int16),
                       f32["logits"].to(torch.bfloat16).view(torch.int16))
    # the lse is the log-sum-exp of exactly these logits
    if got.shape[0]:
        m = got.max(axis=1)
        lse_of = m + np.log(np.exp(got - m[:, None]).sum(axis=1))
        lse = gu.to_np64(f32["lse"])
        assert np.abs(lse_of - lse).max() <= 2e-6 * max(1.0, np.abs(lse).max())
    # the padding columns keep the sentinel
    for o in (f32, b16):
        tail = o["buf"][:, V:]
        assert bool((tail == gu.LOGITS_SENTINEL).all())
    return f32, b16


def test_config1_tiny_fp32():
    _check(fi.make_workload(1))


def test_config2_small_bf16():
    _check(fi.make_workload(2))


@pytest.mark.parametrize("N,H,V", [(600, 264, 1500), (257, 64, 257), (1, 8, 2), (513, 136, 777),
                                   (300, 64, 1024)])
@pytest.mark.parametrize("pad", [0, 1, 8])
def test_ragged_bf16(N, H, V, pad):
    """Rows of any length: 16-byte runs where aligned, element stores where a
    run crosses V or the row length breaks the alignment (pad)."""
    _check(fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + V + pad), pad=pad)


@pytest.mark.parametrize("N,H,V", [(130, 70, 301), (3, 5, 7), (64, 16, 64)])
@pytest.mark.parametrize("pad", [0, 5])
def test_ragged_fp32(N, H, V, pad):
    _check(fi.make_custom(N, H, V, dtype=torch.float32, seed=N + V + pad), pad=pad)


@pytest.mark.parametrize("s", [30.0, 2.0])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_softcap(s, dtype):
    w = fi.make_custom(300, 136, 1000, dtype=dtype, seed=31, w_std=0.5)
    w.softcap = s
    f32, _ = _check(w)
    assert float(f32["logits"].abs().max()) <= s


def test_mean_external_count_scale_and_ignored():
    w = fi.make_custom(700, 128, 1500, dtype=torch.bfloat16, seed=32)
    w.reduction = "mean"
    _check(w, mb_scale=0.375)
    w.labels.fill_(w.ignore_index)
    f32, _ = _check(w)
    assert f32["loss"] == 0.0 and f32["num_tokens"] == 0


def test_empty_batch():
    import lm_head_linear_amd as m
    dev = gu.device()
    W = torch.randn(300, 64, device=dev).to(torch.bfloat16)
    h = torch.empty(0, 64, dtype=torch.bfloat16, device=dev)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    loss, nt, lg = m.flce_forward_logits(h, W, y)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nt.item() == 0 and tuple(lg.shape) == (0, 300)


def test_invalid_label_fails_closed_and_logits_still_written():
    w = fi.make_custom(200, 64, 300, dtype=torch.bfloat16, seed=33)
    w.labels[0, 11] = 300
    f = gu.run_gpu_forward_logits(w)
    assert f["status"] == 5 and np.isnan(f["loss"])
    assert bool((f["logits"] != gu.LOGITS_SENTINEL).all())


def test_misaligned_row_start():
    """A logits buffer that starts 2 bytes past a 16-byte boundary (bf16) or
    4 bytes past (float32): every store goes element by element."""
    import lm_head_linear_amd as m
    dev = gu.device()
    w = fi.make_custom(260, 64, 520, dtype=torch.bfloat16, seed=34)
    h = w.h.reshape(-1, w.H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    base = m.flce_forward_logits(h, W, y)[2]
    for dt in (torch.float32, torch.bfloat16):
        raw = torch.full((260 * 520 + 8,), gu.LOGITS_SENTINEL, dtype=dt, device=dev)
        view = raw[1:1 + 260 * 520].view(260, 520)
        m.flce_forward_logits(h, W, y, logits=view)
        torch.cuda.synchronize()
        assert torch.equal(view.float(), base.to(dt).float())
        assert raw[0].item() == gu.LOGITS_SENTINEL
        assert bool((raw[1 + 260 * 520:] == gu.LOGITS_SENTINEL).all())
