"""Pins of the float64 oracle against facts that do not come from the oracle.

Each test fixes the oracle to a closed form, an invariant, a textbook special
case, brute-force finite differences, or an independent PyTorch CPU float64
cross-entropy, so that a dropped term, a wrong sign or index, or a transposed
operand anywhere in the oracle fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import flce_inputs as fi
from oracle import flce_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
IGN = -100


def _rand_case(N, H, V, seed, ignore=0, w_std=0.5, h_std=1.0):
    rng = np.random.default_rng(seed)
    h = rng.normal(0, h_std, (N, H))
    W = rng.normal(0, w_std, (V, H))
    y = rng.integers(0, V, N)
    if ignore:
        y[rng.permutation(N)[:ignore]] = IGN
    return h, W, y


# ---------------------------------------------------------------- P1 zero W
@pytest.mark.parametrize("V", [1024, 32000])
@pytest.mark.parametrize("softcap", [0.0, 30.0])
@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_zero_weight_closed_form(V, softcap, reduction):
    """W = 0: every logit is 0 (tanh(0) = 0), so each valid token costs log V."""
    rng = np.random.default_rng(1)
    N, H = 24, 16
    h = rng.normal(size=(N, H))
    y = rng.integers(0, V, N)
    y[[3, 7, 11]] = IGN
    n = N - 3
    r = orc.flce_reference(h, np.zeros((V, H)), y, softcap=softcap, reduction=reduction)
    per_tok = math.log(V)
    expect = per_tok * n if reduction == "sum" else per_tok
    assert r.loss64 == pytest.approx(expect, rel=1e-13)
    assert np.all(r.dH == 0.0)
    c = 1.0 if reduction == "sum" else 1.0 / n
    valid = y != IGN
    dW = np.zeros((V, H))
    for i in range(N):
        if valid[i]:
            dW += (1.0 / V) * h[i][None, :]
            dW[y[i]] -= h[i]
    np.testing.assert_allclose(r.dW, c * dW, rtol=1e-12, atol=1e-14)


def test_zero_weight_log_values():
    """The per-token loss at W = 0 for the vocab sizes used here is log V, written
    through the factorisations 1024 = 2^10, 32000 = 2^8 5^3, 131072 = 2^17 and
    256000 = 2^11 5^3."""
    l2, l5 = math.log(2.0), math.log(5.0)
    for V, val in [(1024, 10 * l2), (32000, 8 * l2 + 3 * l5),
                   (131072, 17 * l2), (256000, 11 * l2 + 3 * l5)]:
        r = orc.flce_reference(np.ones((1, 2)), np.zeros((V, 2)), np.array([5]))
        assert r.loss64 == pytest.approx(val, rel=1e-14)


# ---------------------------------------------------------------- P2 zero h
@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_zero_hidden_closed_form(reduction):
    rng = np.random.default_rng(2)
    N, H, V = 10, 6, 37
    W = rng.normal(size=(V, H))
    y = rng.integers(0, V, N)
    y[[0, 4]] = IGN
    n = N - 2
    r = orc.flce_reference(np.zeros((N, H)), W, y, reduction=reduction)
    assert r.loss64 == pytest.approx(math.log(V) * (n if reduction == "sum" else 1), rel=1e-13)
    assert np.all(r.dW == 0.0)
    c = 1.0 if reduction == "sum" else 1.0 / n
    for i in range(N):
        if y[i] == IGN:
            assert np.all(r.dH[i] == 0.0)
        else:
            np.testing.assert_allclose(r.dH[i], c * (W.mean(0) - W[y[i]]), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- P3 all ignored
def test_all_ignored_from_pages_example():
    """The example of an MTP label roll that leaves no target (Ling-3.1-flash
    discussion 7): the loss is 0, not NaN, and so are the gradients."""
    with open(os.path.join(GOLDEN, "empty_targets_after_roll.json")) as f:
        g = json.load(f)
    lab = torch.tensor(g["labels"])
    rolled = torch.roll(lab, shifts=-1)
    assert rolled.tolist() == g["after_roll"]
    shifted = rolled[1:]
    assert shifted.tolist() == g["after_causal_shift"]
    assert bool((shifted == IGN).all())
    rng = np.random.default_rng(3)
    N = shifted.numel()
    h = rng.normal(size=(N, 8))
    W = rng.normal(size=(50, 8))
    for red in ("sum", "mean"):
        r = orc.flce_reference(h, W, shifted.numpy(), reduction=red)
        assert r.loss64 == g["expected"]["loss"] and not math.isnan(r.loss64)
        assert r.num_tokens == g["expected"]["num_tokens"]
        assert np.all(r.dH == 0.0) and np.all(r.dW == 0.0)


def test_empty_batch():
    for red in ("sum", "mean"):
        r = orc.flce_reference(np.zeros((0, 4)), np.ones((9, 4)), np.zeros(0, dtype=np.int64),
                               reduction=red)
        assert r.loss64 == 0.0 and r.num_tokens == 0
        assert r.dH.shape == (0, 4) and np.all(r.dW == 0.0)


# ---------------------------------------------------------------- P4 mean vs sum
def test_mean_equals_sum_over_count():
    h, W, y = _rand_case(40, 12, 90, seed=4, ignore=9)
    s = orc.flce_reference(h, W, y, reduction="sum")
    m = orc.flce_reference(h, W, y, reduction="mean")
    n = 40 - 9
    assert s.num_tokens == n and m.num_tokens == 0
    assert m.loss64 * n == pytest.approx(s.loss64, rel=1e-12)
    np.testing.assert_allclose(m.dH * n, s.dH, rtol=1e-11, atol=1e-15)
    np.testing.assert_allclose(m.dW * n, s.dW, rtol=1e-11, atol=1e-15)


def test_external_count_normalises_sum():
    h, W, y = _rand_case(30, 8, 40, seed=5, ignore=4)
    s = orc.flce_reference(h, W, y, reduction="sum")
    t = orc.flce_reference(h, W, y, reduction="sum", num_label_tokens=52)
    assert t.loss64 == pytest.approx(s.loss64 / 52, rel=1e-13)
    assert t.num_tokens == s.num_tokens == 26
    np.testing.assert_allclose(t.dW * 52, s.dW, rtol=1e-12, atol=1e-15)
    with pytest.raises(ValueError):
        orc.flce_reference(h, W, y, reduction="mean", num_label_tokens=52)
    z = orc.flce_reference(h, W, y, reduction="sum", num_label_tokens=0)
    assert z.loss64 == s.loss64


# ---------------------------------------------------------------- P5 tiny vocab
def test_vocab_one_is_zero():
    rng = np.random.default_rng(6)
    r = orc.flce_reference(rng.normal(size=(5, 3)), rng.normal(size=(1, 3)), np.zeros(5, dtype=int))
    assert r.loss64 == 0.0
    assert np.all(r.dH == 0.0) and np.all(r.dW == 0.0)


@pytest.mark.parametrize("softcap", [0.0, 1.5])
def test_vocab_two_is_logistic(softcap):
    """V = 2: loss = softplus(z_other - z_target); d/dz_target = -sigmoid(z_other - z_target)."""
    rng = np.random.default_rng(7)
    N, H = 9, 4
    h = rng.normal(size=(N, H))
    W = rng.normal(size=(2, H))
    y = rng.integers(0, 2, N)
    r = orc.flce_reference(h, W, y, softcap=softcap)
    Z = h @ W.T
    Zc = softcap * np.tanh(Z / softcap) if softcap else Z
    d = np.array([Zc[i, 1 - y[i]] - Zc[i, y[i]] for i in range(N)])
    softplus = np.logaddexp(0.0, d)
    assert r.loss64 == pytest.approx(softplus.sum(), rel=1e-13)
    # gradient w.r.t. z_target through dH: dH_i = sum_v G_iv W_v with G_i,target = -sigmoid(d)
    sig = 1.0 / (1.0 + np.exp(-d))
    deriv = (1 - np.tanh(Z / softcap) ** 2) if softcap else np.ones_like(Z)
    for i in range(N):
        g = np.zeros(2)
        g[y[i]] = -sig[i]
        g[1 - y[i]] = sig[i]
        g = g * deriv[i]
        np.testing.assert_allclose(r.dH[i], g @ W, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P6 finite differences
def _fd_check(h, W, y, softcap, reduction, rel):
    r = orc.flce_reference(h, W, y, softcap=softcap, reduction=reduction)
    eps = 1e-6

    def f(hh, WW):
        return orc.flce_reference(hh, WW, y, softcap=softcap, reduction=reduction).loss64

    dH = np.zeros_like(h)
    for idx in np.ndindex(*h.shape):
        hp = h.copy(); hp[idx] += eps
        hm = h.copy(); hm[idx] -= eps
        dH[idx] = (f(hp, W) - f(hm, W)) / (2 * eps)
    dW = np.zeros_like(W)
    for idx in np.ndindex(*W.shape):
        Wp = W.copy(); Wp[idx] += eps
        Wm = W.copy(); Wm[idx] -= eps
        dW[idx] = (f(h, Wp) - f(h, Wm)) / (2 * eps)
    scale_h = np.abs(dH).max()
    scale_w = np.abs(dW).max()
    assert np.abs(r.dH - dH).max() <= rel * scale_h
    assert np.abs(r.dW - dW).max() <= rel * scale_w


@pytest.mark.parametrize("softcap", [0.0, 2.0])
@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_finite_differences(softcap, reduction):
    rng = np.random.default_rng(8)
    # W std 1 so that softcap 2 saturates tanh and its derivative matters.
    h = rng.normal(size=(3, 4))
    W = rng.normal(size=(5, 4))
    y = np.array([0, 4, 2])
    _fd_check(h, W, y, softcap, reduction, 1e-7)
    h2 = rng.normal(size=(4, 3))
    W2 = rng.normal(size=(7, 3))
    y2 = np.array([6, IGN, 1, IGN])
    _fd_check(h2, W2, y2, softcap, reduction, 1e-7)


# ---------------------------------------------------------------- P7 softcap
def test_softcap_derivative_by_fd():
    s = 3.0
    z = np.linspace(-5 * s, 5 * s, 101)
    zp, d = orc.softcap_logits(z[None, :], s)
    eps = 1e-6
    fd = (s * np.tanh((z + eps) / s) - s * np.tanh((z - eps) / s)) / (2 * eps)
    # central-difference rounding error is about s * 1e-16 / eps = 3e-10
    np.testing.assert_allclose(d[0], fd, rtol=1e-8, atol=1e-9)
    np.testing.assert_allclose(zp[0], s * np.tanh(z / s), rtol=0, atol=0)
    assert np.all(np.abs(zp) < s)


def test_huge_softcap_is_no_softcap():
    h, W, y = _rand_case(12, 5, 20, seed=9, ignore=2)
    a = orc.flce_reference(h, W, y, softcap=0.0)
    b = orc.flce_reference(h, W, y, softcap=1e8)
    assert b.loss64 == pytest.approx(a.loss64, rel=1e-12)
    np.testing.assert_allclose(b.dH, a.dH, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(b.dW, a.dW, rtol=1e-10, atol=1e-14)


def test_negative_or_nonfinite_softcap_rejected():
    h, W, y = _rand_case(3, 2, 4, seed=10)
    for s in (-1.0, float("inf"), float("nan")):
        with pytest.raises(ValueError):
            orc.flce_reference(h, W, y, softcap=s)


# ---------------------------------------------------------------- P8 invariants
def test_rows_of_gradient_sum_to_zero():
    """Without softcap each row of softmax - onehot sums to 0, so sum_v dW[v] = 0."""
    h, W, y = _rand_case(20, 7, 33, seed=11, ignore=3)
    r = orc.flce_reference(h, W, y)
    assert np.abs(r.dW.sum(0)).max() <= 1e-12 * np.abs(r.dW).max() * 33


def test_shift_invariance():
    """W -> W + 1 b^T adds h.b to every logit of a row: loss and dH unchanged."""
    h, W, y = _rand_case(15, 6, 21, seed=12, ignore=2)
    b = np.random.default_rng(13).normal(size=6)
    a = orc.flce_reference(h, W, y)
    s = orc.flce_reference(h, W + b[None, :], y)
    assert s.loss64 == pytest.approx(a.loss64, rel=1e-12)
    # dH = G W; G unchanged and rows of G sum to 0, so G (1 b^T) = 0.
    np.testing.assert_allclose(s.dH, a.dH, rtol=1e-9, atol=1e-12)


def test_token_permutation():
    h, W, y = _rand_case(18, 5, 25, seed=14, ignore=4)
    p = np.random.default_rng(15).permutation(18)
    a = orc.flce_reference(h, W, y)
    b = orc.flce_reference(h[p], W, y[p])
    assert b.loss64 == pytest.approx(a.loss64, rel=1e-13)
    np.testing.assert_allclose(b.dH, a.dH[p], rtol=1e-13, atol=0)
    np.testing.assert_allclose(b.dW, a.dW, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- P9 library cross-check
@pytest.mark.parametrize("softcap", [0.0, 2.5])
@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_against_torch_cpu_float64_cross_entropy(softcap, reduction):
    """An independent float64 PyTorch CPU cross-entropy with autograd."""
    h, W, y = _rand_case(37, 16, 101, seed=16, ignore=6, w_std=0.7)
    r = orc.flce_reference(h, W, y, softcap=softcap, reduction=reduction)
    th = torch.tensor(h, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    logits = F.linear(th, tW)
    if softcap:
        logits = softcap * torch.tanh(logits / softcap)
    loss = F.cross_entropy(logits, torch.tensor(y), ignore_index=IGN, reduction=reduction)
    loss.backward()
    assert r.loss64 == pytest.approx(loss.item(), rel=1e-12)
    np.testing.assert_allclose(r.dH, th.grad.numpy(), rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(r.dW, tW.grad.numpy(), rtol=1e-10, atol=1e-14)
    lse = torch.logsumexp(logits.detach(), dim=1).numpy()
    np.testing.assert_allclose(r.lse, lse, rtol=1e-13)


def test_mean_of_all_ignored_differs_from_torch_nan():
    """PyTorch's 'mean' over an empty target set is NaN; the clamped count gives 0."""
    h, W, _ = _rand_case(4, 3, 6, seed=17)
    y = np.full(4, IGN)
    t = F.cross_entropy(torch.tensor(h) @ torch.tensor(W).T, torch.tensor(y),
                        ignore_index=IGN, reduction="mean")
    assert math.isnan(t.item())
    assert orc.flce_reference(h, W, y, reduction="mean").loss64 == 0.0


def test_invalid_label_raises():
    h, W, y = _rand_case(5, 3, 6, seed=18)
    y[2] = 6
    with pytest.raises(ValueError):
        orc.flce_reference(h, W, y)
    y[2] = -1
    with pytest.raises(ValueError):
        orc.flce_reference(h, W, y)
    y[2] = IGN
    orc.flce_reference(h, W, y)


def test_ignore_index_inside_vocab():
    """ignore_index is matched by equality, also when it names a vocab row."""
    h, W, y = _rand_case(12, 4, 9, seed=19)
    y[:4] = 3
    r = orc.flce_reference(h, W, y, ignore_index=3)
    keep = y != 3
    s = orc.flce_reference(h[keep], W, y[keep])
    assert r.loss64 == pytest.approx(s.loss64, rel=1e-13)
    assert np.all(r.dH[~keep] == 0.0)


# ---------------------------------------------------------------- P10 construction counts
@pytest.mark.parametrize("k,n", [(1, 29), (2, 1946), (3, 6144), (4, 7373), (5, 15872)])
def test_construction_counts(k, n):
    lab, ignored = fi.make_labels(k)
    valid = orc.valid_mask(lab.numpy(), fi.IGNORE_INDEX)
    assert orc.count_valid(valid) == n
    assert lab.numel() - ignored == n


def test_config1_num_tokens_and_loss_order():
    w = fi.make_workload(1)
    r = orc.flce_reference(w.h.reshape(-1, w.H).numpy(), w.W.numpy(), w.labels.reshape(-1).numpy())
    assert r.num_tokens == 29
    # Small W: every logit is near 0, the loss per token is near log V.
    assert abs(r.loss64 / 29 - math.log(1024)) < 0.1


# ---------------------------------------------------------------- P11 micro-batches
@pytest.mark.parametrize("reduction", ["sum", "mean"])
def test_micro_batch_additivity(reduction):
    h, W, y = _rand_case(64, 8, 30, seed=20, ignore=11)
    n = int((y != IGN).sum())
    T = n if reduction == "sum" else None
    full = orc.flce_reference(h, W, y, reduction=reduction, num_label_tokens=T)
    loss = 0.0
    dW = np.zeros_like(W)
    for mb in range(4):
        s = slice(16 * mb, 16 * (mb + 1))
        n_mb = int((y[s] != IGN).sum())
        scale = orc.micro_batch_scale(n_mb, n, reduction)
        r = orc.flce_reference(h[s], W, y[s], reduction=reduction, num_label_tokens=T,
                               mb_scale=scale)
        loss += r.loss64
        dW += r.dW
        np.testing.assert_allclose(r.dH, full.dH[s], rtol=1e-12, atol=1e-16)
    assert loss == pytest.approx(full.loss64, rel=1e-12)
    np.testing.assert_allclose(dW, full.dW, rtol=1e-11, atol=1e-15)


def test_forward_rows_and_dW_rows_match_full():
    h, W, y = _rand_case(26, 6, 19, seed=21, ignore=5)
    for s in (0.0, 1.3):
        full = orc.flce_reference(h, W, y, softcap=s, reduction="mean")
        lse, tok, _ = orc.forward_rows(h, W, y, IGN, s, row_chunk=7)
        np.testing.assert_allclose(lse, full.lse, rtol=1e-14)
        np.testing.assert_allclose(tok, full.token_loss, rtol=1e-14)
        rows = np.array([0, 5, 18])
        dw = orc.dW_rows(h, W, y, lse, rows, c=full.c, softcap=s)
        np.testing.assert_allclose(dw, full.dW[rows], rtol=1e-11, atol=1e-15)
        toks = np.array([1, 4, 25])
        dh = orc.dH_rows(h[toks], W, y[toks], lse[toks], c=full.c, softcap=s)
        np.testing.assert_allclose(dh, full.dH[toks], rtol=1e-11, atol=1e-15)


# ---------------------------------------------------------------- logits output
def test_logits_rows_brute_force():
    """Each logit as a plain sum of products over the hidden dimension (exact
    fsum) and the cap through math.tanh, element by element: catches a
    transposed operand or a cap applied to the wrong quantity."""
    h, W, _ = _rand_case(3, 5, 4, seed=41)
    for s in (0.0, 0.7):
        Z = orc.logits_rows(h, W, s)
        assert Z.shape == (3, 4)
        for i in range(3):
            for v in range(4):
                z = math.fsum(h[i, k] * W[v, k] for k in range(5))
                if s > 0:
                    z = s * math.tanh(z / s)
                assert abs(Z[i, v] - z) <= 1e-14 * max(1.0, abs(z)), (i, v, s)


def test_logits_rows_closed_forms():
    # one-hot hidden state picks a column of W; the cap of atanh(1/2) with
    # s = 1 is exactly 1/2
    W = np.array([[0.25, -3.0], [2.0, 0.5], [-1.5, 1.0]])
    Z = orc.logits_rows(np.array([[0.0, 1.0]]), W, 0.0)
    np.testing.assert_array_equal(Z, [[-3.0, 0.5, 1.0]])
    Z = orc.logits_rows(np.array([[math.atanh(0.5)]]), np.array([[1.0], [-1.0]]), 1.0)
    np.testing.assert_allclose(Z, [[0.5, -0.5]], rtol=0, atol=1e-15)
    assert not orc.logits_rows(np.ones((2, 3)), np.zeros((5, 3)), 2.0).any()


def test_logits_rows_feed_the_loss():
    """The logits are the ones the loss is formed from: their log-sum-exp is
    the lse of the forward, the target entry the target logit, and the capped
    values lie strictly inside (-s, s)."""
    h, W, y = _rand_case(40, 12, 37, seed=42, ignore=6, w_std=2.0)
    for s in (0.0, 3.0):
        Z = orc.logits_rows(h, W, s)
        lse, tok, zt = orc.forward_rows(h, W, y, IGN, s)
        m = Z.max(axis=1)
        np.testing.assert_allclose(m + np.log(np.exp(Z - m[:, None]).sum(axis=1)), lse,
                                   rtol=1e-14)
        valid = y != IGN
        np.testing.assert_allclose(Z[valid, y[valid]], zt[valid], rtol=1e-15)
        np.testing.assert_allclose(lse[valid] - Z[valid, y[valid]], tok[valid], rtol=1e-12)
        if s > 0:
            assert np.abs(Z).max() < s
