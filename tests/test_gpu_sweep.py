"""A second seeded sweep of random shapes against the oracle, across every
entry point at once: bf16 and float32 gradients, dW added to an existing one,
the no-recompute variant, the forward-only and logits-returning forwards;
even and odd hidden sizes; 0-95% ignored tokens; softcaps; an external count;
micro-batch scales 1, 0.5 and 0; several vocabulary chunk sizes."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
import oracle.flce_oracle as orc
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
MODES = ["step", "f32grad", "nr", "forward", "logits", "step_acc"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lm_head_linear_amd._lib as L
    L.load()
    yield


@pytest.mark.parametrize("k", range(120))
def test_sweep_case(k, monkeypatch):
    rng = np.random.default_rng(50000 + k)
    N, V = int(rng.integers(1, 900)), int(rng.integers(1, 3000))
    H = int(rng.integers(1, 48)) * 8 + (int(rng.integers(1, 8)) if k % 2 else 0)
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=50000 + k,
                       w_std=float(rng.choice([0.02, 0.3])),
                       ignore_frac=float(rng.choice([0.0, 0.1, 0.5, 0.95])),
                       labels=str(rng.choice(["uniform", "zipf"])),
                       softcap=float(rng.choice([0.0, 0.0, 2.0, 30.0])),
                       reduction=str(rng.choice(["sum", "mean"])))
    if w.reduction == "sum" and rng.random() < 0.3:
        w.num_label_tokens = int(rng.integers(1, 3 * N + 2))
    mode = MODES[k % len(MODES)]
    vchunk = int(rng.choice([0, 256, 512, 768]))
    if vchunk:
        monkeypatch.setenv("FLCE_VCHUNK", str(vchunk))
    mb = float(rng.choice([1.0, 0.5, 0.0]))
    print(f"case {k}: N={N} H={H} V={V} s={w.softcap} {w.reduction} T={w.num_label_tokens} "
          f"mode={mode} vchunk={vchunk} mb={mb}", flush=True)
    r = gu.run_oracle(w, mb_scale=mb)
    if mode in ("forward", "logits"):
        f = (gu.run_gpu_forward(w, mb_scale=mb) if mode == "forward"
             else gu.run_gpu_forward_logits(w, mb_scale=mb, pad=k % 3))
        assert f["status"] == 0 and f["num_tokens"] == r.num_tokens
        gu.assert_loss(f["loss"], r.loss64)
        assert np.abs(gu.to_np64(f["lse"]) - r.lse).max() <= 1e-5 * max(1.0, np.abs(r.lse).max())
        if mode == "logits":
            Z = orc.logits_rows(w.h.reshape(-1, w.H).to(torch.float64).numpy(),
                                w.W.to(torch.float64).numpy(), w.softcap)
            assert (np.abs(gu.to_np64(f["logits"]) - Z) <= gu.logits_tolerance(w)).all()
        return
    if mode == "step_acc":
        dW0 = (torch.randn(V, H, generator=torch.Generator().manual_seed(k)) * 0.05).to(torch.bfloat16)
        g = gu.run_gpu(w, mb_scale=mb, dW=dW0.to(gu.device()), accumulate_dW=True)
        assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
        gu.assert_loss(g["loss"], r.loss64)
        gu.assert_grad("dW", g["dW"], r.dW + dW0.to(torch.float64).numpy(), gu.GRAD_TOL[torch.bfloat16])
        gu.assert_grad("dH", g["dH"], r.dH, gu.GRAD_TOL[torch.bfloat16])
        return
    kw = {}
    if mode == "f32grad":
        kw["grad_dtype"] = torch.float32
    if mode == "nr":
        kw.update(recompute=False, token_chunk=int(rng.choice([0, 256, 512])))
    g = gu.run_gpu(w, mb_scale=mb, **kw)
    if mode == "f32grad":
        assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
        gu.assert_loss(g["loss"], r.loss64)
        gu.assert_grad("dH", g["dH"], r.dH, gu.GRAD_TOL[torch.float32])
        gu.assert_grad("dW", g["dW"], r.dW, gu.GRAD_TOL[torch.float32])
    else:
        gu.assert_parity(w, g, r)
