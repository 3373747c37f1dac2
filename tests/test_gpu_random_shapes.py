"""Seeded random sweep of small problems against the float64 oracle: ragged
token counts, hidden sizes and vocabularies, both dtypes and reductions, the
softcap, forced vocabulary chunks, and each entry point (the full step, float32
gradients, the no-recompute variant with small token chunks, the forward
only, the forward with logits), at the tolerances the other parity tests
use."""
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


def _case(k):
    rng = np.random.default_rng(5000 + k)
    dtype = torch.float32 if k % 7 == 0 else torch.bfloat16
    N = int(rng.integers(1, 700))
    H = int(rng.integers(1, 40)) * 8 if dtype == torch.bfloat16 else int(rng.integers(1, 200))
    V = int(rng.integers(1, 2500))
    w = fi.make_custom(N, H, V, dtype=dtype, seed=6000 + k, w_std=float(rng.choice([0.02, 0.3])),
                       ignore_frac=float(rng.choice([0.0, 0.1, 0.5])),
                       labels=str(rng.choice(["uniform", "zipf"])))
    w.reduction = str(rng.choice(["sum", "mean"]))
    if rng.random() < 0.3:
        w.softcap = float(rng.choice([2.0, 30.0]))
    if w.reduction == "sum" and rng.random() < 0.3:
        w.num_label_tokens = int(rng.integers(1, 3 * N + 2))
    mode = ["step", "step", "f32grad", "nr", "forward"][k % 5] if dtype == torch.bfloat16 else "step"
    if mode == "forward" and k % 10 == 9:
        mode = "logits"
    vchunk = int(rng.choice([0, 256, 512])) if mode in ("step", "f32grad") else 0
    tchunk = int(rng.choice([0, 256])) if mode == "nr" else 0
    mb = float(rng.choice([1.0, 0.5]))
    return w, mode, vchunk, tchunk, mb


@pytest.mark.parametrize("k", range(100))
def test_random_case(k, monkeypatch):
    w, mode, vchunk, tchunk, mb = _case(k)
    if vchunk:
        monkeypatch.setenv("FLCE_VCHUNK", str(vchunk))
    print(f"case {k}: N={w.N} H={w.H} V={w.V} {w.dtype} {w.reduction} s={w.softcap} "
          f"T={w.num_label_tokens} mode={mode} vchunk={vchunk} tchunk={tchunk} mb={mb}", flush=True)
    r = gu.run_oracle(w, mb_scale=mb)
    if mode == "forward":
        f = gu.run_gpu_forward(w, mb_scale=mb)
        assert f["status"] == 0 and f["num_tokens"] == r.num_tokens
        gu.assert_loss(f["loss"], r.loss64)
        assert np.abs(gu.to_np64(f["lse"]) - r.lse).max() <= 1e-5 * max(1.0, np.abs(r.lse).max())
        return
    if mode == "logits":
        ldt = torch.bfloat16 if k % 20 == 19 else torch.float32
        f = gu.run_gpu_forward_logits(w, logits_dtype=ldt, pad=k % 3, mb_scale=mb)
        assert f["status"] == 0 and f["num_tokens"] == r.num_tokens
        gu.assert_loss(f["loss"], r.loss64)
        assert np.abs(gu.to_np64(f["lse"]) - r.lse).max() <= 1e-5 * max(1.0, np.abs(r.lse).max())
        Z = orc.logits_rows(w.h.reshape(-1, w.H).to(torch.float64).numpy(),
                            w.W.to(torch.float64).numpy(), w.softcap)
        tol = gu.logits_tolerance(w)
        if ldt == torch.bfloat16:   # plus half a bf16 unit in the last place
            tol = tol * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(Z)
        assert (np.abs(gu.to_np64(f["logits"]) - Z) <= tol).all()
        assert bool((f["buf"][:, w.V:] == gu.LOGITS_SENTINEL).all())
        return
    kw = {}
    if mode == "f32grad":
        kw["grad_dtype"] = torch.float32
    if mode == "nr":
        kw.update(recompute=False, token_chunk=tchunk)
    g = gu.run_gpu(w, mb_scale=mb, **kw)
    if mode == "f32grad":
        assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
        gu.assert_loss(g["loss"], r.loss64)
        gu.assert_grad("dH", g["dH"], r.dH, gu.GRAD_TOL[torch.float32])
        gu.assert_grad("dW", g["dW"], r.dW, gu.GRAD_TOL[torch.float32])
    else:
        gu.assert_parity(w, g, r)
