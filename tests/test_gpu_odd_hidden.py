"""bf16 inputs with a hidden size that is not a multiple of 8 (the NeMo
linear_ce page, "API", puts no limit on the hidden size of hidden_states):
the call runs at the width rounded up to 8 on zero-padded copies in its
workspace. GPU parity against the float64 oracle for every entry point that
gathers (bf16 and float32 gradients, the no-recompute variant, forward only),
with ignored tokens, a softcap, several vocabulary and token chunks and an
accumulated dW; and bit-identity with the same call made on inputs the
caller padded with zeros, for the forwards that do not gather too."""
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


def _padded(w: fi.Workload) -> fi.Workload:
    """The same problem with h and W zero-padded to a multiple of 8 columns."""
    Hp = -(-w.H // 8) * 8
    h = torch.zeros(*w.h.shape[:-1], Hp, dtype=w.h.dtype)
    h[..., :w.H] = w.h
    W = torch.zeros(w.V, Hp, dtype=w.W.dtype)
    W[:, :w.H] = w.W
    return fi.Workload(name=w.name + "_padded", h=h, W=W, labels=w.labels,
                       ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction,
                       num_label_tokens=w.num_label_tokens, micro_batches=w.micro_batches,
                       expected_valid=w.expected_valid, std_w=w.std_w)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _same_as_padded(w, g, gp):
    """The odd-width call equals the caller-padded one bit for bit."""
    assert g["status"] == 0 and gp["status"] == 0
    assert g["num_tokens"] == gp["num_tokens"]
    assert _bits(g["loss_t"]).item() == _bits(gp["loss_t"]).item()
    if g.get("lse") is not None:
        assert torch.equal(_bits(g["lse"]), _bits(gp["lse"]))
    for k in ("dH", "dW"):
        if k in g:
            assert g[k].shape[-1] == w.H
            assert torch.equal(_bits(g[k]), _bits(gp[k][:, :w.H].contiguous())), k
            assert bool((gp[k][:, w.H:] == 0).all()), k     # the pad columns stay zero


@pytest.mark.parametrize("N,H,V,chunk,cap,red", [
    (300, 100, 1000, 0, 0.0, "sum"),          # one chunk
    (777, 61, 1500, 256, 30.0, "mean"),       # many chunks, softcap
    (520, 1, 700, 512, 0.0, "sum"),           # H = 1
    (1100, 4095, 900, 512, 0.0, "sum"),       # wide rows, 2 chunks
])
def test_odd_hidden_step(N, H, V, chunk, cap, red, vchunk):
    if chunk:
        vchunk(chunk)
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + H, ignore_frac=0.2,
                       softcap=cap, reduction=red)
    g = gu.run_gpu(w)
    gu.assert_parity(w, g, gu.run_oracle(w))
    _same_as_padded(w, g, gu.run_gpu(_padded(w)))


@pytest.mark.parametrize("N,H,V", [(300, 100, 1000), (777, 61, 1500)])
def test_odd_hidden_float32_gradients(N, H, V, vchunk):
    vchunk(256)
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=N + H + 1, ignore_frac=0.1,
                       softcap=30.0)
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
    _same_as_padded(w, g, gu.run_gpu(_padded(w), grad_dtype=torch.float32))


@pytest.mark.parametrize("token_chunk", [0, 256])
def test_odd_hidden_no_recompute(token_chunk):
    w = fi.make_custom(700, 100, 1300, dtype=torch.bfloat16, seed=41, ignore_frac=0.15)
    g = gu.run_gpu(w, recompute=False, token_chunk=token_chunk)
    gu.assert_parity(w, g, gu.run_oracle(w))
    _same_as_padded(w, g, gu.run_gpu(_padded(w), recompute=False, token_chunk=token_chunk))


def test_odd_hidden_forward_only():
    w = fi.make_custom(900, 100, 1300, dtype=torch.bfloat16, seed=42, ignore_frac=0.3,
                       softcap=20.0, reduction="mean")
    f = gu.run_gpu_forward(w)
    r = gu.run_oracle(w)
    assert f["status"] == 0 and f["num_tokens"] == r.num_tokens
    gu.assert_loss(f["loss"], r.loss64)
    lse = gu.to_np64(f["lse"])
    assert np.abs(lse - r.lse).max() <= 1e-5 * max(1.0, np.abs(r.lse).max())
    b = gu.run_gpu(w)                       # the full call's forward, bit for bit
    assert _bits(f["loss_t"]).item() == _bits(b["loss_t"]).item()
    assert torch.equal(_bits(f["lse"]), _bits(b["lse"]))
    _same_as_padded(w, f, gu.run_gpu_forward(_padded(w)))


def test_odd_hidden_accumulated_dW(vchunk):
    """dW added to the caller's: the padded copy starts from it."""
    import lm_head_linear_amd as m
    vchunk(512)
    w = fi.make_custom(600, 100, 1300, dtype=torch.bfloat16, seed=43, ignore_frac=0.1)
    dev = gu.device()
    dW0 = (torch.randn(w.V, w.H, generator=torch.Generator().manual_seed(5)) * 0.1).to(torch.bfloat16)
    g = gu.run_gpu(w, dW=dW0.to(dev), accumulate_dW=True)
    r = gu.run_oracle(w)
    ref = r.dW + dW0.to(torch.float64).numpy()
    gu.assert_grad("dW", g["dW"], ref, gu.GRAD_TOL[torch.bfloat16])
    wp = _padded(w)
    dW0p = torch.zeros(w.V, wp.H, dtype=torch.bfloat16)
    dW0p[:, :w.H] = dW0
    gp = gu.run_gpu(wp, dW=dW0p.to(dev), accumulate_dW=True)
    _same_as_padded(w, g, gp)


def test_odd_hidden_accumulated_float32_dW(vchunk):
    """float32 dW added to the caller's at an odd width: the padded float32
    copy starts from it."""
    vchunk(256)
    w = fi.make_custom(500, 61, 1100, dtype=torch.bfloat16, seed=45, ignore_frac=0.2, softcap=30.0)
    dev = gu.device()
    dW0 = torch.randn(w.V, w.H, generator=torch.Generator().manual_seed(6)) * 0.1
    g = gu.run_gpu(w, dW=dW0.to(dev), accumulate_dW=True, grad_dtype=torch.float32)
    r = gu.run_oracle(w)
    gu.assert_grad("dW", g["dW"], r.dW + dW0.to(torch.float64).numpy(), gu.GRAD_TOL[torch.float32])
    gu.assert_grad("dH", g["dH"], r.dH, gu.GRAD_TOL[torch.float32])
    wp = _padded(w)
    dW0p = torch.zeros(w.V, wp.H)
    dW0p[:, :w.H] = dW0
    gp = gu.run_gpu(wp, dW=dW0p.to(dev), accumulate_dW=True, grad_dtype=torch.float32)
    _same_as_padded(w, g, gp)


@pytest.mark.parametrize("cap", [0.0, 30.0])
def test_odd_hidden_logits_and_noalloc(cap):
    """The two forwards that do not gather (logits-returning, allocation-free)
    read a padded copy of h: the same bits as on caller-padded inputs, and as
    flce_forward."""
    import lm_head_linear_amd as m
    w = fi.make_custom(300, 100, 700, dtype=torch.bfloat16, seed=44, ignore_frac=0.2, softcap=cap)
    wp = _padded(w)
    for dt in (torch.float32, torch.bfloat16):
        a = gu.run_gpu_forward_logits(w, logits_dtype=dt)
        b = gu.run_gpu_forward_logits(wp, logits_dtype=dt)
        assert a["status"] == 0 and b["status"] == 0
        assert _bits(a["loss_t"]).item() == _bits(b["loss_t"]).item()
        assert torch.equal(_bits(a["lse"]), _bits(b["lse"]))
        assert torch.equal(_bits(a["logits"]), _bits(b["logits"]))
    f = gu.run_gpu_forward(w)
    assert _bits(f["loss_t"]).item() == _bits(a["loss_t"]).item()
    r = gu.run_oracle(w)
    gu.assert_loss(f["loss"], r.loss64)
    dev = gu.device()
    h, W, y = w.h.reshape(-1, w.H).to(dev), w.W.to(dev), w.labels.reshape(-1).to(dev)
    loss = torch.empty((), device=dev)
    nt = torch.empty((), dtype=torch.int64, device=dev)
    lse = torch.empty(w.N, device=dev)
    m.flce_forward_noalloc(h, W, y, ignore_index=w.ignore_index, softcap=w.softcap,
                           reduction=w.reduction, loss=loss, num_tokens=nt, lse_out=lse)
    torch.cuda.synchronize()
    assert _bits(loss).item() == _bits(f["loss_t"]).item()
    assert torch.equal(_bits(lse), _bits(f["lse"]))


@pytest.mark.parametrize("k", range(20))
def test_odd_hidden_random(k, monkeypatch):
    """Seeded random shapes with H % 8 != 0 over the gathering entry points."""
    rng = np.random.default_rng(7100 + k)
    N, V = int(rng.integers(1, 700)), int(rng.integers(1, 2500))
    H = int(rng.integers(0, 40)) * 8 + int(rng.integers(1, 8))
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=7100 + k,
                       ignore_frac=float(rng.choice([0.0, 0.1, 0.5])),
                       softcap=float(rng.choice([0.0, 30.0])),
                       reduction=str(rng.choice(["sum", "mean"])))
    mode = ["step", "f32grad", "nr", "forward"][k % 4]
    if mode in ("step", "f32grad"):
        monkeypatch.setenv("FLCE_VCHUNK", str(int(rng.choice([0, 256, 512]))))
    print(f"case {k}: N={N} H={H} V={V} s={w.softcap} {w.reduction} mode={mode}", flush=True)
    r = gu.run_oracle(w)
    if mode == "forward":
        f = gu.run_gpu_forward(w)
        assert f["status"] == 0 and f["num_tokens"] == r.num_tokens
        gu.assert_loss(f["loss"], r.loss64)
        return
    if mode == "f32grad":
        g = gu.run_gpu(w, grad_dtype=torch.float32)
        assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
        gu.assert_loss(g["loss"], r.loss64)
        gu.assert_grad("dH", g["dH"], r.dH, gu.GRAD_TOL[torch.float32])
        gu.assert_grad("dW", g["dW"], r.dW, gu.GRAD_TOL[torch.float32])
        return
    g = gu.run_gpu(w, recompute=mode != "nr", token_chunk=int(rng.choice([0, 256])))
    gu.assert_parity(w, g, r)
