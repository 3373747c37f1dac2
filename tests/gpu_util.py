"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same seeded values, compare to the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import flce_inputs as fi
from oracle import flce_oracle as orc

# Tolerances (written here, used by every parity test):
#   loss       |gpu - ref| <= 1e-5 * |ref|   (exactly 0 when ref is 0)
#   bf16 grads max|gpu - ref| <= 2e-2 * max|ref| per tensor
#   fp32 grads max|gpu - ref| <= 1e-4 * max|ref| per tensor
#   num_tokens bit-exact; ignored rows of dH exactly zero
#   logits     per element, the float32 rounding-error bound of logits_tolerance;
#              bf16 logits bit-equal to the round-to-nearest-even of float32 ones
LOSS_RTOL = 1e-5
GRAD_TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def device():
    return torch.device("cuda:0")


def to_np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def run_gpu(w: fi.Workload, *, mb_scale=1.0, lse=True, dev=None, **kw):
    import lm_head_linear_amd as m
    dev = dev or device()
    H = w.H
    h = w.h.reshape(-1, H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    lse_out = torch.full((h.shape[0],), float("nan"), dtype=torch.float32, device=dev) if lse else None
    status = torch.full((), -1, dtype=torch.int32, device=dev)
    args = dict(ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction,
                num_label_tokens=w.num_label_tokens, mb_scale=mb_scale, lse_out=lse_out,
                status=status)
    args.update(kw)
    loss, nt, dH, dW = m.flce_forward_backward(h, W, y, **args)
    torch.cuda.synchronize(dev)
    return dict(loss=float(loss.item()), loss_t=loss, num_tokens=int(nt.item()), dH=dH, dW=dW,
                lse=lse_out, status=int(status.item()))


def run_gpu_forward(w: fi.Workload, *, mb_scale=1.0, dev=None, **kw):
    """The forward-only entry on the same inputs: loss, num_tokens, lse, status."""
    import lm_head_linear_amd as m
    dev = dev or device()
    h = w.h.reshape(-1, w.H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    lse_out = torch.full((h.shape[0],), float("nan"), dtype=torch.float32, device=dev)
    status = torch.full((), -1, dtype=torch.int32, device=dev)
    args = dict(ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction,
                num_label_tokens=w.num_label_tokens, mb_scale=mb_scale, lse_out=lse_out,
                status=status)
    args.update(kw)
    loss, nt = m.flce_forward(h, W, y, **args)
    torch.cuda.synchronize(dev)
    return dict(loss=float(loss.item()), loss_t=loss, num_tokens=int(nt.item()), lse=lse_out,
                status=int(status.item()))


def run_oracle(w: fi.Workload, *, mb_scale=1.0, **kw):
    h = w.h.reshape(-1, w.H).to(torch.float64).numpy()
    W = w.W.to(torch.float64).numpy()
    y = w.labels.reshape(-1).numpy()
    args = dict(ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction,
                num_label_tokens=w.num_label_tokens, mb_scale=mb_scale)
    args.update(kw)
    return orc.flce_reference(h, W, y, **args)


def assert_loss(gpu_loss: float, ref: float, rtol: float = LOSS_RTOL):
    if ref == 0.0:
        assert gpu_loss == 0.0, f"loss {gpu_loss} != exact 0"
    else:
        err = abs(gpu_loss - ref)
        assert err <= rtol * abs(ref), f"loss {gpu_loss} vs ref {ref}: rel err {err / abs(ref):.3e}"


def assert_grad(name: str, gpu: torch.Tensor, ref: np.ndarray, tol: float) -> float:
    """Every element within tol * max|ref|; returns max err / max|ref|."""
    g = to_np64(gpu)
    assert g.shape == ref.shape, (name, g.shape, ref.shape)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(g - ref).max()) if ref.size else 0.0
    if scale == 0.0:
        assert err == 0.0, f"{name}: reference is zero, max |gpu| = {err}"
        return 0.0
    assert err <= tol * scale, f"{name}: max err {err:.3e} > {tol} * {scale:.3e} (ratio {err / scale:.3e})"
    return err / scale


def assert_parity(w: fi.Workload, g: dict, r, *, check_lse=True):
    tol = GRAD_TOL[w.dtype]
    assert g["status"] == 0
    assert g["num_tokens"] == r.num_tokens
    assert_loss(g["loss"], r.loss64)
    eh = assert_grad("dH", g["dH"], r.dH, tol)
    ew = assert_grad("dW", g["dW"], r.dW, tol)
    rel = abs(g["loss"] - r.loss64) / abs(r.loss64) if r.loss64 else 0.0
    print(f"PARITY {w.name} N={r.dH.shape[0]} H={w.H} V={w.V}: loss rel={rel:.2e} "
          f"dH max err/max ref={eh:.2e} dW max err/max ref={ew:.2e}", flush=True)
    y = w.labels.reshape(-1).numpy()
    ign = y == w.ignore_index
    if ign.any():
        dh = g["dH"][torch.from_numpy(np.flatnonzero(ign)).to(g["dH"].device)]
        assert bool((dh == 0).all()), "ignored rows of dH must be exactly zero"
    if check_lse and g["lse"] is not None and r.lse.size:
        lse = to_np64(g["lse"])
        err = np.abs(lse - r.lse).max()
        assert err <= 1e-5 * max(1.0, np.abs(r.lse).max()), f"lse max err {err:.3e}"


def run_gpu_forward_logits(w: fi.Workload, *, logits_dtype=torch.float32, pad=0, mb_scale=1.0,
                           dev=None, **kw):
    """The logits-returning forward entry on the same inputs. The logits go to
    a [N, V + pad] buffer prefilled with a sentinel, through its [N, V] view;
    returns loss, num_tokens, lse, status, the view and the whole buffer."""
    import lm_head_linear_amd as m
    dev = dev or device()
    h = w.h.reshape(-1, w.H).to(dev)
    W = w.W.to(dev)
    y = w.labels.reshape(-1).to(dev)
    N, V = h.shape[0], W.shape[0]
    buf = torch.full((N, V + pad), LOGITS_SENTINEL, dtype=logits_dtype, device=dev)
    view = buf[:, :V]
    lse_out = torch.full((N,), float("nan"), dtype=torch.float32, device=dev)
    status = torch.full((), -1, dtype=torch.int32, device=dev)
    args = dict(ignore_index=w.ignore_index, softcap=w.softcap, reduction=w.reduction,
                num_label_tokens=w.num_label_tokens, mb_scale=mb_scale, lse_out=lse_out,
                status=status, logits=view)
    args.update(kw)
    loss, nt, lg = m.flce_forward_logits(h, W, y, **args)
    torch.cuda.synchronize(dev)
    assert lg.data_ptr() == view.data_ptr()
    return dict(loss=float(loss.item()), loss_t=loss, num_tokens=int(nt.item()), lse=lse_out,
                status=int(status.item()), logits=view, buf=buf)


LOGITS_SENTINEL = -12288.0     # -1.5 * 2^13: exact in float32 and bfloat16


def logits_tolerance(w: fi.Workload, rows=None) -> np.ndarray:
    """Per-element bound on |GPU logit - float64 logit| for the float32 logits.

    The kernels accumulate the H products of a logit in float32 (bf16 x bf16
    products are exact in float32, float32 ones round once). The worst-case
    bound, about H u sum_k |p_k| (u = 2^-24), is far too loose to notice a
    dropped product. The test uses the rounding-error model instead: with
    independent rounding errors, summing H terms of random sign errs by a
    standard deviation of about u H rms(p) / sqrt(6), since the partial sums
    grow like sqrt(k) rms(p). The bound is 8 u H rms(p) = 8 u sqrt(H sum_k
    p_k^2), about 20 standard deviations, while one missing or doubled
    product errs by |p_k|, near rms(p) itself. With a softcap the hyperbolic
    tangent (from the hardware exp2 and reciprocal) adds an absolute error of a
    few 1e-7 times s, bounded by 1e-6 s; the cap's slope is at most 1, so the
    product error passes through it unamplified.
    """
    h2 = np.square(w.h.reshape(-1, w.H).to(torch.float64).numpy())
    if rows is not None:
        h2 = h2[rows]
    W2 = np.square(w.W.to(torch.float64).numpy())
    tol = 8.0 * 2.0 ** -24 * np.sqrt(w.H * (h2 @ W2.T))
    if w.softcap > 0:
        tol = tol + 1e-6 * w.softcap
    return tol + 1e-30
