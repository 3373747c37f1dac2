"""CPU check of the logits tolerance the GPU parity tests use: it accepts a
sequential float32 accumulation of the same products (what the kernels do,
in some order) and rejects a logit that misses one product or counts one
twice, on the sizes and value laws of those tests."""
import numpy as np
import pytest
import torch

import flce_inputs as fi
from tests import gpu_util as gu


def _f32_sequential(h, W):
    """Logits by a float32 running sum over k, for all elements at once."""
    h32 = h.astype(np.float32)
    W32 = W.astype(np.float32)
    acc = np.zeros((h.shape[0], W.shape[0]), dtype=np.float32)
    for k in range(h.shape[1]):
        acc = (acc + np.outer(h32[:, k], W32[:, k]).astype(np.float32)).astype(np.float32)
    return acc.astype(np.float64)


@pytest.mark.parametrize("N,H,V,dtype,w_std", [
    (64, 1024, 512, torch.bfloat16, 0.02),
    (40, 264, 700, torch.bfloat16, 0.5),
    (50, 70, 301, torch.float32, 0.02),
])
def test_tolerance_accepts_float32_and_rejects_a_dropped_product(N, H, V, dtype, w_std):
    w = fi.make_custom(N, H, V, dtype=dtype, seed=H + V, w_std=w_std)
    h = w.h.reshape(-1, H).to(torch.float64).numpy()
    W = w.W.to(torch.float64).numpy()
    Z = h @ W.T
    tol = gu.logits_tolerance(w)
    f32 = _f32_sequential(h, W)
    assert (np.abs(f32 - Z) <= tol).all()
    assert (np.abs(f32 - Z) / tol).max() < 0.5          # a wide margin
    rng = np.random.default_rng(0)
    for k in rng.choice(H, 4, replace=False):
        p = np.outer(h[:, k], W[:, k])
        for bad in (Z - p, Z + p):
            frac = (np.abs(bad - Z) > tol).mean()
            assert frac > 0.9, (k, frac)       # almost every logit notices it
