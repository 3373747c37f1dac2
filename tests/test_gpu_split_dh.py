"""Split-K dH against the float64 oracle. When the dH GEMM's N x H output has
fewer than 128 tiles of 256 x 256, its K (the vocabulary rows of a chunk, or
the whole vocabulary in the no-recompute variant) is split into segments
whose float32 partial products a fixed-order reduction adds up, after the
running sum of the earlier chunks. These shapes are ragged in every
dimension, have K long enough to split, and cover one chunk, several chunks
(the running sum), float32 gradients (never split) and the no-recompute
variant, at the tolerances of the other parity tests."""
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


CASES = [
    # N, H, V, vchunk, softcap, reduction, mode
    (300, 136, 9000, 0, 0.0, "sum", "step"),          # one chunk, 4 segments
    (600, 264, 20000, 4096, 0.0, "mean", "step"),     # 5 chunks, 2 segments each
    (257, 64, 12345, 0, 30.0, "sum", "step"),         # softcap, ragged segments
    (300, 136, 9000, 0, 0.0, "sum", "f32grad"),       # float32 gradients: not split
    (300, 136, 9000, 0, 0.0, "sum", "nr"),            # no-recompute: K = V split
    (1000, 512, 8200, 0, 0.0, "mean", "nr"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}-{c[6]}-vc{c[3]}" for c in CASES])
def test_split_dh(case, monkeypatch):
    N, H, V, vchunk, softcap, reduction, mode = case
    if vchunk:
        monkeypatch.setenv("FLCE_VCHUNK", str(vchunk))
    w = fi.make_custom(N, H, V, dtype=torch.bfloat16, seed=9100 + N, w_std=0.3,
                       ignore_frac=0.1, labels="uniform")
    w.reduction = reduction
    w.softcap = softcap
    print(f"split dH case N={N} H={H} V={V} vchunk={vchunk} s={softcap} {reduction} {mode}",
          flush=True)
    r = gu.run_oracle(w)
    kw = {}
    if mode == "f32grad":
        kw["grad_dtype"] = torch.float32
    if mode == "nr":
        kw.update(recompute=False)
    g = gu.run_gpu(w, **kw)
    if mode == "f32grad":
        assert g["status"] == 0 and g["num_tokens"] == r.num_tokens
        gu.assert_loss(g["loss"], r.loss64)
        gu.assert_grad("dH", g["dH"], r.dH, gu.GRAD_TOL[torch.float32])
        gu.assert_grad("dW", g["dW"], r.dW, gu.GRAD_TOL[torch.float32])
    else:
        gu.assert_parity(w, g, r)
