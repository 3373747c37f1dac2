"""The bf16 backward runs over the non-ignored tokens only, gathered in order
(their G rows are the only non-zero ones). GPU parity against the oracle for
ignore patterns that stress the gather: masked prefixes of every sequence,
runs across 256-token tile edges, a single kept token, ignored first and last
tokens, over several backward chunks and with a split-K dH; the rows of
ignored tokens in dH are exactly zero even when dH held NaN before the call;
an all-ignored call leaves an accumulated dW bit for bit unchanged; the same
patterns with float32 gradients."""
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


def _mask(N, kind, rng):
    m = np.zeros(N, dtype=bool)
    if kind == "prefix":                  # first quarter of each of 2 sequences
        S = N // 2
        m[:S // 4] = True
        m[S:S + S // 4] = True
    elif kind == "tile_edges":            # runs across the 256-token tile edges
        for e in range(256, N, 256):
            m[max(0, e - 37):e + 21] = True
    elif kind == "one_kept":
        m[:] = True
        m[N // 3] = False
    elif kind == "ends":
        m[0] = m[N - 1] = True
        m[rng.choice(N, N // 5, replace=False)] = True
    elif kind == "random_half":
        m[rng.choice(N, N // 2, replace=False)] = True
    return m


@pytest.mark.parametrize("kind", ["prefix", "tile_edges", "one_kept", "ends", "random_half"])
@pytest.mark.parametrize("N,H,V,chunk", [
    (1100, 264, 3000, 1024),    # 3 chunks, ragged everywhere, split-K dH (few tiles)
    (2048, 512, 2560, 0),       # one chunk
    (777, 128, 1500, 256),      # many chunks
])
def test_compact_patterns(kind, N, H, V, chunk, vchunk):
    if chunk:
        vchunk(chunk)
    rng = np.random.default_rng(N + V)
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + H, ignore_frac=0.0,
                       softcap=30.0 if kind == "ends" else 0.0,
                       reduction="mean" if kind == "prefix" else "sum")
    w.labels.view(-1)[torch.from_numpy(_mask(N, kind, rng))] = fi.IGNORE_INDEX
    dev = gu.device()
    dH = torch.full((N, H), float("nan"), dtype=torch.bfloat16, device=dev)
    g = gu.run_gpu(w, dH=dH)
    r = gu.run_oracle(w)
    gu.assert_parity(w, g, r)              # includes: ignored rows of dH exactly 0


@pytest.mark.parametrize("kind", ["tile_edges", "one_kept", "ends"])
@pytest.mark.parametrize("N,H,V,chunk", [
    (1100, 264, 3000, 1024),    # 3 chunks, ragged everywhere
    (777, 128, 1500, 256),      # many chunks
])
def test_compact_patterns_f32grad(kind, N, H, V, chunk, vchunk):
    """float32 gradients over the gathered tokens: dH is its own float32
    running sum at the tokens' original rows."""
    vchunk(chunk)
    rng = np.random.default_rng(N + V + 1)
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + H + 1, ignore_frac=0.0,
                       softcap=30.0 if kind == "ends" else 0.0, reduction="sum")
    w.labels.view(-1)[torch.from_numpy(_mask(N, kind, rng))] = fi.IGNORE_INDEX
    dev = gu.device()
    dH = torch.full((N, H), float("nan"), dtype=torch.float32, device=dev)
    g = gu.run_gpu(w, dH=dH, grad_dtype=torch.float32)
    r = gu.run_oracle(w)
    assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
    gu.assert_loss(g["loss"], r.loss64)
    tol = gu.GRAD_TOL[torch.float32]
    gu.assert_grad("dH", g["dH"], r.dH, tol)
    gu.assert_grad("dW", g["dW"], r.dW, tol)
    ign = torch.from_numpy(np.flatnonzero(w.labels.reshape(-1).numpy() == w.ignore_index))
    assert bool((g["dH"][ign.to(dev)] == 0).all())


def test_all_ignored_keeps_accumulated_dW(vchunk):
    import lm_head_linear_amd as m
    vchunk(512)
    w = fi.make_custom(600, 128, 1300, dtype=torch.bfloat16, seed=31, ignore_frac=1.0)
    dev = gu.device()
    h, W = w.h.reshape(-1, w.H).to(dev), w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    dW0 = torch.randn(W.shape, device=dev).to(torch.bfloat16)
    dW = dW0.clone()
    dH = torch.full(h.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    loss, nt, dH, dW = m.flce_forward_backward(h, W, y, dH=dH, dW=dW, accumulate_dW=True)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and nt.item() == 0
    assert bool((dH == 0).all())
    assert torch.equal(dW.view(torch.int16), dW0.view(torch.int16))


def test_compact_equals_on_two_calls_with_different_masks(vchunk):
    """The gather's workspace from an earlier call (another mask) does not
    leak into the next one."""
    vchunk(512)
    w = fi.make_custom(900, 136, 2000, dtype=torch.bfloat16, seed=32, ignore_frac=0.6)
    g1 = gu.run_gpu(w)
    w2 = fi.make_custom(900, 136, 2000, dtype=torch.bfloat16, seed=32, ignore_frac=0.05)
    g2 = gu.run_gpu(w2)
    gu.assert_parity(w2, g2, gu.run_oracle(w2))
    gu.assert_parity(w, g1, gu.run_oracle(w))


@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_forward_skips_ignored_tokens_without_changing_a_bit(cap, vchunk):
    """Without per-token lse the forward runs over the kept tokens only; with
    it, over all of them. Loss, dH and dW are bit-identical either way, and
    the loss equals the forward-only entry's (per-token losses are summed by
    original position), with the oracle agreeing."""
    import lm_head_linear_amd as m
    vchunk(512)
    w = fi.make_custom(1500, 264, 2100, dtype=torch.bfloat16, seed=33, ignore_frac=0.0,
                       softcap=cap, reduction="mean")
    w.labels[:, :300] = fi.IGNORE_INDEX                   # masked prefix
    w.labels[0, 700:777] = fi.IGNORE_INDEX
    a = gu.run_gpu(w, lse=False)
    b = gu.run_gpu(w, lse=True)
    f = gu.run_gpu_forward(w)
    assert a["loss_t"].view(torch.int32).item() == b["loss_t"].view(torch.int32).item()
    assert a["loss_t"].view(torch.int32).item() == f["loss_t"].view(torch.int32).item()
    assert torch.equal(b["lse"].view(torch.int32), f["lse"].view(torch.int32))
    for k in ("dH", "dW"):
        assert torch.equal(a[k].view(torch.int16), b[k].view(torch.int16)), k
    # the forward-only entry without lse_out (its GEMM over the kept tokens)
    import lm_head_linear_amd as m
    dev = gu.device()
    lf, nf = m.flce_forward(w.h.reshape(-1, w.H).to(dev), w.W.to(dev), w.labels.reshape(-1).to(dev),
                            ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction)
    torch.cuda.synchronize()
    assert lf.view(torch.int32).item() == a["loss_t"].view(torch.int32).item()
    assert nf.item() == a["num_tokens"]
    r = gu.run_oracle(w)
    gu.assert_parity(w, b, r)
    gu.assert_parity(w, a, r, check_lse=False)


@pytest.mark.parametrize("N", [20000, 70000])
@pytest.mark.parametrize("entry", ["step", "step_lse", "no_recompute", "forward"])
def test_long_gather(N, entry):
    """Gathers over many tokens: 20000 is three passes of the one-workgroup
    label scan and gather (8192 tokens a pass, the last one ragged), 70000 is
    past its limit (65536) and runs the multi-block count and placement. A
    third of the tokens ignored at random plus a masked prefix; dH starts as
    NaN, so an ignored row that is not zeroed fails."""
    import lm_head_linear_amd as m
    rng = np.random.default_rng(N)
    w = fi.make_custom(N, 64, 300, dtype=torch.bfloat16, seed=N, ignore_frac=0.0, softcap=0.0,
                       reduction="sum")
    mask = np.zeros(N, dtype=bool)
    mask[rng.choice(N, N // 3, replace=False)] = True
    mask[:1000] = True
    w.labels.view(-1)[torch.from_numpy(mask)] = fi.IGNORE_INDEX
    r = gu.run_oracle(w)
    assert r.num_tokens == int((~mask).sum())
    dev = gu.device()
    if entry == "forward":
        g = gu.run_gpu_forward(w)
        assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
        gu.assert_loss(g["loss"], r.loss64)
        lse = gu.to_np64(g["lse"])
        assert np.abs(lse - r.lse).max() <= 1e-5 * max(1.0, np.abs(r.lse).max())
        return
    dH = torch.full((N, w.H), float("nan"), dtype=torch.bfloat16, device=dev)
    if entry == "no_recompute":
        h = w.h.reshape(N, w.H).to(dev)
        status = torch.full((), -1, dtype=torch.int32, device=dev)
        loss, nt, dH, dW = m.flce_forward_backward_nr(h, w.W.to(dev), w.labels.reshape(N).to(dev),
                                                      ignore_index=w.ignore_index, dH=dH,
                                                      status=status, token_chunk=8192)
        torch.cuda.synchronize()
        g = dict(loss=float(loss.item()), num_tokens=int(nt.item()), dH=dH, dW=dW, lse=None,
                 status=int(status.item()))
    else:
        g = gu.run_gpu(w, lse=entry == "step_lse", dH=dH)
    gu.assert_parity(w, g, r)              # includes: ignored rows of dH exactly 0
