"""GPU parity at the full sizes of the large-vocab, softcapped and long
configurations, in the launch configuration the benchmark times (one call,
default vocabulary chunk), against the float64 oracle on identical values.

The oracle runs the whole forward once per configuration (every token's lse
and loss, so the summed loss and every per-token lse are compared in full);
dH is compared on sampled tokens and dW on sampled vocabulary rows, which the
oracle computes one by one from its own lse. Counts are compared exactly and
every ignored row of dH must be exactly zero. The long configuration is also
run as 4 micro-batches with a shared external token count and dW
accumulation.
"""
import math

import numpy as np
import pytest
import torch

import flce_inputs as fi
from oracle import flce_oracle as orc
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

_CACHE = {}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_linear_amd._lib as L
    L.load()
    yield
    _CACHE.clear()


def _case(k):
    """Workload k, its float64 views and the oracle's forward (cached)."""
    if k not in _CACHE:
        w = fi.make_workload(k)
        h64 = w.h.reshape(-1, w.H).to(torch.float64).numpy()
        W64 = w.W.to(torch.float64).numpy()
        y = w.labels.reshape(-1).numpy()
        lse, tok, _ = orc.forward_rows(h64, W64, y, w.ignore_index, w.softcap)
        _CACHE.clear()          # keep one configuration's float64 copies at a time
        _CACHE[k] = (w, h64, W64, y, lse, tok)
    return _CACHE[k]


def _sample_tokens(N, y, ign, rng):
    picks = {0, 1, 255, 256, 257, N // 2, N - 257, N - 256, N - 1}
    picks.update(rng.choice(N, 40, replace=False).tolist())
    ignored = np.flatnonzero(y == ign)
    if ignored.size:
        picks.update(ignored[:4].tolist())
    return np.array(sorted(p for p in picks if 0 <= p < N))


def _sample_vocab(V, y, ign, chunk, rng):
    picks = {0, 1, 2, 255, 256, V // 2, V - 256, V - 1, chunk - 1, chunk, chunk + 1}
    vals, cnt = np.unique(y[y != ign], return_counts=True)
    picks.update(vals[np.argsort(-cnt)[:6]].tolist())          # most frequent targets
    picks.update(rng.choice(V, 24, replace=False).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < V))


def _check(k, g, *, T=None, mb_scale=1.0, label="", tol=2e-2):
    w, h64, W64, y, lse, tok = _case(k)
    n = int((y != w.ignore_index).sum())
    assert n == w.expected_valid
    T = w.num_label_tokens if T is None else T
    c = orc.scale_factor(n, w.reduction, T, mb_scale)
    loss_ref = c * math.fsum(tok.tolist())
    print(f"{label} loss gpu={g['loss']:.9g} ref={loss_ref:.9g}", flush=True)
    gu.assert_loss(g["loss"], loss_ref)
    assert g["num_tokens"] == orc.num_tokens_for(n, w.reduction)
    if g.get("lse") is not None:
        d = np.abs(gu.to_np64(g["lse"]) - lse).max()
        assert d <= 1e-5 * max(1.0, np.abs(lse).max()), f"lse max err {d}"
    rng = np.random.default_rng(k)
    import lm_head_linear_amd as m
    chunk = m.flce_vocab_chunk(w.N, w.H, w.V, w.dtype, g["dW"].dtype)
    toks = _sample_tokens(w.N, y, w.ignore_index, rng)
    ref_dh = orc.dH_rows(h64[toks], W64, y[toks], lse[toks], c=c, ignore_index=w.ignore_index,
                         softcap=w.softcap)
    gu.assert_grad("dH rows", g["dH"][torch.from_numpy(toks).to(g["dH"].device)], ref_dh, tol)
    rows = _sample_vocab(w.V, y, w.ignore_index, chunk, rng)
    ref_dw = orc.dW_rows(h64, W64, y, lse, rows, c=c, ignore_index=w.ignore_index,
                         softcap=w.softcap)
    gu.assert_grad("dW rows", g["dW"][torch.from_numpy(rows).to(g["dW"].device)], ref_dw, tol)
    ign = torch.from_numpy(np.flatnonzero(y == w.ignore_index)).to(g["dH"].device)
    if ign.numel():
        assert bool((g["dH"][ign] == 0).all()), "ignored rows of dH must be exactly zero"
    assert bool(torch.isfinite(g["dW"].float()).all())


def _forward_only_matches(w, g):
    """The forward-only entry returns the same loss, count and lse bits."""
    f = gu.run_gpu_forward(w)
    assert f["loss_t"].view(torch.int32).item() == g["loss_t"].view(torch.int32).item()
    assert f["num_tokens"] == g["num_tokens"] and f["status"] == g["status"] == 0
    assert torch.equal(f["lse"].view(torch.int32), g["lse"].view(torch.int32))


def test_large_vocab_full():
    w = _case(3)[0]
    g = gu.run_gpu(w)
    assert g["num_tokens"] == 0          # 'mean'
    _check(3, g, label="large_vocab")
    _forward_only_matches(w, g)


def test_large_vocab_float32_gradients():
    """Float32 dH and dW for the bf16 large-vocab inputs, at the float32
    tolerance on the sampled rows."""
    w = _case(3)[0]
    g = gu.run_gpu(w, grad_dtype=torch.float32)
    assert g["dH"].dtype == torch.float32 and g["num_tokens"] == 0
    _check(3, g, label="large_vocab f32 grads", tol=1e-4)


def test_large_vocab_no_recompute():
    """The no-recompute variant at full size, in 2 token chunks of 4096."""
    w = _case(3)[0]
    g = gu.run_gpu(w, recompute=False, token_chunk=4096)
    assert g["num_tokens"] == 0
    _check(3, g, label="large_vocab no recompute")


def _forward_logits_check(k, label):
    """The logits-returning forward at full size: loss, count and lse the same
    bits as the forward-only entry; float32 logits of sampled tokens against
    the oracle's Z' row by row; every row's lse the log-sum-exp of its stored
    logits; the bf16 logits the round-to-nearest-even of the float32 ones."""
    w, h64, W64, y, lse, tok = _case(k)
    N, V = h64.shape[0], W64.shape[0]
    f = gu.run_gpu_forward(w)
    print(f"{label}: float32 logits [{N}, {V}]", flush=True)
    g = gu.run_gpu_forward_logits(w, logits_dtype=torch.float32)
    assert g["loss_t"].view(torch.int32).item() == f["loss_t"].view(torch.int32).item()
    assert g["num_tokens"] == f["num_tokens"] and g["status"] == f["status"] == 0
    assert torch.equal(g["lse"].view(torch.int32), f["lse"].view(torch.int32))
    lg = g["logits"]
    rng = np.random.default_rng(k + 100)
    rows = _sample_tokens(N, y, w.ignore_index, rng)
    Z = orc.logits_rows(h64[rows], W64, w.softcap)
    got = lg[torch.as_tensor(rows, device=lg.device)].double().cpu().numpy()
    err = np.abs(got - Z)
    tol = gu.logits_tolerance(w, rows)
    assert (err <= tol).all(), f"max err/tol {(err / tol).max():.3f}"
    print(f"{label}: sampled logits max err {err.max():.3e} (max tol ratio "
          f"{(err / tol).max():.3f})", flush=True)
    worst = 0.0
    for r0 in range(0, N, 1024):
        blk = lg[r0:r0 + 1024].double()
        lse_of = torch.logsumexp(blk, dim=1)
        worst = max(worst, float((lse_of - g["lse"][r0:r0 + 1024].double()).abs().max()))
    assert worst <= 2e-6 * max(1.0, float(np.abs(lse).max())), worst
    b16 = lg.to(torch.bfloat16)
    del g, lg
    torch.cuda.empty_cache()
    print(f"{label}: bf16 logits", flush=True)
    gb = gu.run_gpu_forward_logits(w, logits_dtype=torch.bfloat16)
    assert gb["loss_t"].view(torch.int32).item() == f["loss_t"].view(torch.int32).item()
    assert torch.equal(gb["logits"].view(torch.int16), b16.view(torch.int16))
    del gb, b16
    torch.cuda.empty_cache()


def test_large_vocab_forward_logits():
    _forward_logits_check(3, "large_vocab")


def test_softcapped_forward_logits():
    _forward_logits_check(4, "softcapped")


def test_softcapped_full():
    w = _case(4)[0]
    g = gu.run_gpu(w)
    _check(4, g, label="softcapped")
    _forward_only_matches(w, g)


def test_softcapped_no_recompute():
    """No-recompute variant with the softcap at full size (one chunk of 8192
    tokens, V = 256000: the softcap derivative rebuilt from the stored
    probabilities)."""
    w = _case(4)[0]
    g = gu.run_gpu(w, recompute=False)
    _check(4, g, label="softcapped no recompute")


def test_long_full_and_external_count():
    w = _case(5)[0]
    g = gu.run_gpu(w)
    _check(5, g, label="long T=15872")
    # the count is the one used: twice the count halves loss and gradients
    g2 = gu.run_gpu(w, num_label_tokens=2 * w.num_label_tokens)
    _check(5, g2, T=2 * w.num_label_tokens, label="long T=31744")


def test_long_no_recompute():
    """No-recompute variant on 16384 tokens: 2 token chunks, dW added up over
    them, with the external count."""
    w = _case(5)[0]
    g = gu.run_gpu(w, recompute=False)
    _check(5, g, label="long no recompute")


def test_long_four_micro_batches():
    """4 micro-batches of 4096 flattened tokens (the ignored span crosses the
    boundary between the second and third), shared external count, dW added
    up across calls: equal to the single call over the whole batch."""
    import lm_head_linear_amd as m
    w = _case(5)[0]
    dev = gu.device()
    N, H = w.N, w.H
    h = w.h.reshape(N, H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(N).to(dev)
    dH = torch.empty_like(h)
    dW = torch.empty_like(W)
    T = w.num_label_tokens
    total, ntok = 0.0, 0
    mb = N // 4
    for i in range(4):
        s = slice(i * mb, (i + 1) * mb)
        loss, nt, _, _ = m.flce_forward_backward(h[s], W, y[s], ignore_index=w.ignore_index,
                                                 reduction=w.reduction, num_label_tokens=T,
                                                 mb_scale=m.micro_batch_scale(0, 0, "sum"),
                                                 dH=dH[s], dW=dW, accumulate_dW=i > 0)
        total += loss.item()
        ntok += nt.item()
    torch.cuda.synchronize()
    assert ntok == T
    _check(5, dict(loss=total, num_tokens=ntok, dH=dH, dW=dW, lse=None), label="long 4 mb")
