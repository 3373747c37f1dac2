"""GPU parity at the full sizes of the large-vocab, softcapped and long
configurations, in the launch configuration the benchmark times (one call,
default vocabulary chunk), against the float64 oracle on identical values.

The oracle runs the whole forward and backward once per configuration
(flce_reference: every token's lse and loss, the whole dH and the whole dW),
cached while that configuration's tests run, so every element of loss, lse,
dH and dW is compared: dH and dW within 2e-2 max|ref| per tensor (1e-4 for
float32 gradients). Counts are compared exactly and every ignored row of dH
must be exactly zero. The long configuration is also run as 4 micro-batches
with a shared external token count and dW accumulation, and in the
no-recompute variant with 32 token chunks (dW summed over them in float32).
"""
import math
import time

import numpy as np
import pytest
import torch

import flce_inputs as fi
from oracle import flce_oracle as orc
from tests import gpu_util as gu

# the float64 oracle takes tens of seconds per configuration on the host
pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(900)]

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
    """Workload k, its float64 views and the oracle's whole result (cached,
    one configuration at a time)."""
    if k not in _CACHE:
        _CACHE.clear()
        w = fi.make_workload(k)
        h64 = w.h.reshape(-1, w.H).to(torch.float64).numpy()
        W64 = w.W.to(torch.float64).numpy()
        y = w.labels.reshape(-1).numpy()
        t0 = time.perf_counter()
        r = orc.flce_reference(h64, W64, y, ignore_index=w.ignore_index, softcap=w.softcap,
                               reduction=w.reduction, num_label_tokens=w.num_label_tokens)
        print(f"oracle {w.name}: whole forward + backward in {time.perf_counter() - t0:.1f} s",
              flush=True)
        _CACHE[k] = (w, h64, W64, y, r)
    return _CACHE[k]


def _sample_tokens(N, y, ign, rng):
    """Token rows whose float32 logits are compared one by one with the
    oracle's: tile edges, random rows and a few ignored ones."""
    picks = {0, 1, 255, 256, 257, N // 2, N - 257, N - 256, N - 1}
    picks.update(rng.choice(N, 40, replace=False).tolist())
    ignored = np.flatnonzero(y == ign)
    if ignored.size:
        picks.update(ignored[:4].tolist())
    return np.array(sorted(p for p in picks if 0 <= p < N))


def _max_err(name, gpu, ref, tol, rows=8192):
    """max |gpu - ref| over every element, in row blocks (host memory), against
    tol * max |ref|; returns the ratio err / max |ref|."""
    scale = float(np.abs(ref).max())
    err = 0.0
    for r0 in range(0, ref.shape[0], rows):
        g = gpu[r0:r0 + rows].to("cpu", torch.float64).numpy()
        err = max(err, float(np.abs(g - ref[r0:r0 + rows]).max()))
    assert scale > 0.0, name
    assert err <= tol * scale, f"{name}: max err {err:.3e} > {tol} * {scale:.3e}"
    return err / scale


def _check(k, g, *, T=None, mb_scale=1.0, label="", tol=2e-2):
    w, h64, W64, y, r = _case(k)
    n = int((y != w.ignore_index).sum())
    assert n == w.expected_valid == r.n_valid
    T = w.num_label_tokens if T is None else T
    c = orc.scale_factor(n, w.reduction, T, mb_scale)
    ratio = c / r.c                 # loss and gradients are linear in c
    loss_ref = c * math.fsum(r.token_loss.tolist())
    gu.assert_loss(g["loss"], loss_ref)
    assert g["num_tokens"] == orc.num_tokens_for(n, w.reduction)
    if g.get("lse") is not None:
        d = np.abs(gu.to_np64(g["lse"]) - r.lse).max()
        assert d <= 1e-5 * max(1.0, np.abs(r.lse).max()), f"lse max err {d}"
    eh = _max_err("dH", g["dH"], r.dH * ratio, tol)
    ew = _max_err("dW", g["dW"], r.dW * ratio, tol)
    ign = torch.from_numpy(np.flatnonzero(y == w.ignore_index)).to(g["dH"].device)
    if ign.numel():
        assert bool((g["dH"][ign] == 0).all()), "ignored rows of dH must be exactly zero"
    print(f"PARITY {label}: loss gpu={g['loss']:.9g} ref={loss_ref:.9g} "
          f"rel={abs(g['loss'] - loss_ref) / abs(loss_ref):.2e} "
          f"dH max err/max ref={eh:.2e} dW max err/max ref={ew:.2e}", flush=True)


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
    """Float32 dH and dW for the bf16 large-vocab inputs, every element at the
    float32 tolerance."""
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
    w, h64, W64, y, r = _case(k)
    lse = r.lse
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
    them in float32, with the external count."""
    w = _case(5)[0]
    g = gu.run_gpu(w, recompute=False)
    _check(5, g, label="long no recompute")


def test_long_no_recompute_32_chunks():
    """No-recompute variant in 32 token chunks of 512: each chunk's dW is
    added to a float32 running sum and bf16 is rounded once at the end (the
    chunked path of Modalities PR 464, "What the reference implementations
    do", accumulates gradients in float32), so the error does not grow with
    the chunk count."""
    import lm_head_linear_amd as m
    w = _case(5)[0]
    assert m.flce_token_chunk_nr(w.N, w.H, w.V, w.dtype, 512) == 512
    g = gu.run_gpu(w, recompute=False, token_chunk=512)
    _check(5, g, label="long no recompute 32 chunks")


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


def _gpu_inputs(w):
    dev = gu.device()
    return (w.h.reshape(w.N, w.H).to(dev), w.W.to(dev), w.labels.reshape(w.N).to(dev))


def test_large_vocab_bitwise_deterministic():
    """Two full-size steps on the same inputs give the same bits: no atomics,
    fixed-order sums."""
    import lm_head_linear_amd as m
    w = fi.make_workload(3)
    h, W, y = _gpu_inputs(w)
    outs = []
    for _ in range(2):
        lse = torch.empty(w.N, dtype=torch.float32, device=h.device)
        loss, nt, dH, dW = m.flce_forward_backward(h, W, y, ignore_index=w.ignore_index,
                                                   reduction=w.reduction, lse_out=lse)
        torch.cuda.synchronize()
        outs.append((loss, nt, dH, dW, lse))
    a, b = outs
    assert a[0].view(torch.int32).item() == b[0].view(torch.int32).item()
    assert a[1].item() == b[1].item()
    for x, z in zip(a[2:], b[2:]):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           z.view(torch.int16) if z.dtype == torch.bfloat16 else z.view(torch.int32))


@pytest.mark.parametrize("k", [3, 4, 5])
def test_peak_extra_memory(k):
    """Device memory the call adds on top of its inputs and outputs (the
    workspace) stays at or below N V 4 / 8, an eighth of the float32 logits
    the fused path avoids (Modalities PR 464, "Memory note": 8 GiB at
    [2, 8192, 131072])."""
    import lm_head_linear_amd as m
    w = fi.make_workload(k)
    h, W, y = _gpu_inputs(w)
    dH, dW = torch.empty_like(h), torch.empty_like(W)
    loss = torch.empty((), dtype=torch.float32, device=h.device)
    nt = torch.empty((), dtype=torch.int64, device=h.device)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    m.flce_forward_backward(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                            reduction=w.reduction, num_label_tokens=w.num_label_tokens,
                            dH=dH, dW=dW, loss=loss, num_tokens=nt)
    torch.cuda.synchronize()
    extra = torch.cuda.max_memory_allocated() - base
    bound = w.N * w.V * 4 // 8
    print(f"{w.name}: peak extra device memory {extra / 2**20:.1f} MiB "
          f"(bound {bound / 2**20:.0f} MiB, float32 logits {w.N * w.V * 4 / 2**30:.2f} GiB)",
          flush=True)
    assert 0 < extra <= bound
    assert torch.isfinite(loss).item()
