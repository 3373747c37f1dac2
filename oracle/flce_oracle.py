"""Float64 CPU oracle for fused linear cross-entropy -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this module. The library path never routes through it and it
shares no code with the GPU kernels.

What it computes (plain definition, materialised logits, float64 throughout):

* logits ``Z = h @ W.T`` -- the LM-head projection. The fused loss never forms
  the logits (LlamaFactory error page "cross_entropy and
  fused_linear_cross_entropy cannot both be enabled", section "What it means");
  this oracle is the materialising side, one block of token rows at a time.
* optional softcap ``Z' = s * tanh(Z / s)``, ``s = 0`` meaning off (NeMo
  AutoModel ``linear_ce`` page, API, ``logit_softcapping``), applied to the
  same logits that feed the log-sum-exp and the target gather (twinkle PR 335,
  "PR information", item 3: the fallback must apply the same softcap).
* token-level cross-entropy with ``ignore_index`` (default -100, NeMo API),
  summed over non-ignored tokens in floating point wider than the inputs
  (Modalities PR 464, "What the reference implementations do": the
  sum-over-valid formulation with IGNORE_INDEX on up-cast logits).
* reduction ``'sum'`` or ``'mean'`` (NeMo API ``reduction``); a sum-reduced
  loss may be normalised by an external global count ``num_label_tokens``
  (NeMo API, ``forward`` parameter of that name).
* ``num_tokens`` = count of non-ignored tokens for ``'sum'`` and 0 for
  ``'mean'`` (twinkle PR 335, "PR information", item 1).
* micro-batch scale ``mb_scale`` multiplies the loss and gradients (twinkle PR
  335, item 2: the token-weighted scale, 1.0 for ``'sum'``).
* an empty target set gives loss 0 and zero gradients, via the clamped count
  ``max(n, 1)`` (Ling-3.1-flash discussion 7, "Why use num_items_in_batch for
  MTP?").
* gradients of the returned loss: ``G = c * valid * (softmax(Z') - onehot(y))
  * dZ'/dZ``, ``dH = G @ W``, ``dW = G.T @ h``.
* the logits themselves, ``Z'``, for a caller that needs them (LlamaFactory
  error page, "Source" and "Solutions": ``require_logits`` switches the fused
  loss off because it never forms them).

Readings taken where the pages leave a step open are listed in the project's
design notes; the ones that change arithmetic here: the empty-target rule is
applied to both reductions; ``num_label_tokens`` with ``'mean'`` is an error;
``num_label_tokens <= 0`` means absent; a non-ignored label outside [0, V) is an
error (``ValueError``).

Pins: every function here is checked by the CPU tests against closed forms,
invariants, finite differences, special cases that reduce to textbook
formulas, and an independent float64 PyTorch CPU cross-entropy. No function in
this file is "parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "OracleResult",
    "valid_mask",
    "count_valid",
    "scale_factor",
    "softcap_logits",
    "logsumexp_rows",
    "forward_rows",
    "logits_rows",
    "grad_logits_rows",
    "flce_reference",
    "dW_rows",
    "dH_rows",
    "micro_batch_scale",
]


@dataclass
class OracleResult:
    loss64: float            # the loss in float64
    loss32: float            # the same rounded to float32 (the returned dtype)
    num_tokens: int
    n_valid: int
    c: float                 # the per-token gradient/loss scale
    dH: np.ndarray           # [N, H] float64
    dW: np.ndarray           # [V, H] float64
    lse: np.ndarray          # [N] float64, log-sum-exp of the (softcapped) logits
    token_loss: np.ndarray   # [N] float64, 0 on ignored tokens


def valid_mask(labels: np.ndarray, ignore_index: int) -> np.ndarray:
    """Tokens whose label differs from ``ignore_index`` take part (NeMo API)."""
    return np.asarray(labels) != ignore_index


def count_valid(valid: np.ndarray) -> int:
    """Exact count of non-ignored tokens (twinkle PR 335, item 1)."""
    return int(np.count_nonzero(valid))


def check_labels(labels: np.ndarray, valid: np.ndarray, V: int) -> None:
    """A non-ignored label must name a vocabulary row."""
    bad = valid & ((labels < 0) | (labels >= V))
    if np.any(bad):
        i = int(np.flatnonzero(bad)[0])
        raise ValueError(f"label {int(labels[i])} at token {i} outside [0, {V})")


def scale_factor(n_valid: int, reduction: str, num_label_tokens: Optional[int],
                 mb_scale: float = 1.0) -> float:
    """The factor c with loss = c * (sum of per-token losses over valid tokens).

    * 'sum' without an external count: c = mb_scale (the plain summed loss; the
      micro-batch scale is 1.0 for 'sum', twinkle PR 335 item 2).
    * 'sum' with num_label_tokens = T > 0: c = mb_scale / T (NeMo API: the global
      count normalises a sum-reduced loss).
    * 'mean': c = mb_scale / max(n, 1) -- the clamped count makes an empty
      target set give 0 instead of NaN (Ling-3.1-flash discussion 7).
    """
    T = num_label_tokens if (num_label_tokens is not None and num_label_tokens > 0) else None
    if reduction == "sum":
        return mb_scale / T if T is not None else mb_scale
    if reduction == "mean":
        if T is not None:
            raise ValueError("num_label_tokens normalises a 'sum' loss; not valid with 'mean'")
        return mb_scale / max(n_valid, 1)
    raise ValueError(f"unknown reduction {reduction!r}")


def num_tokens_for(n_valid: int, reduction: str) -> int:
    """twinkle PR 335, item 1: 'mean' returns 0, 'sum' the non-ignored count."""
    return n_valid if reduction == "sum" else 0


def softcap_logits(Z: np.ndarray, softcap: float):
    """Return (Z', dZ'/dZ): s*tanh(Z/s) and 1 - tanh(Z/s)**2; identity when s = 0."""
    if softcap < 0 or not math.isfinite(softcap):
        raise ValueError("softcap must be finite and >= 0")
    if softcap == 0.0:
        return Z, None
    t = np.tanh(Z / softcap)
    return softcap * t, 1.0 - t * t


def logsumexp_rows(Zp: np.ndarray) -> np.ndarray:
    """log(sum_v exp(Z'_v)) per row, shifted by the row max for range safety."""
    m = np.max(Zp, axis=1)
    return m + np.log(np.sum(np.exp(Zp - m[:, None]), axis=1))


def forward_rows(h: np.ndarray, W: np.ndarray, labels: np.ndarray, ignore_index: int,
                 softcap: float, row_chunk: int = 1024):
    """Per-token (lse, loss, target logit) for every row of h, in float64.

    The loss of token i is lse_i - Z'_{i, y_i} on non-ignored tokens and 0 on
    ignored ones. Rows are processed ``row_chunk`` at a time; each row's values
    depend only on that row.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64)
    N = h.shape[0]
    valid = valid_mask(labels, ignore_index)
    check_labels(labels, valid, W.shape[0])
    lse = np.zeros(N)
    tok = np.zeros(N)
    zt = np.zeros(N)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        Zp, _ = softcap_logits(h[r0:r1] @ W.T, softcap)
        l = logsumexp_rows(Zp)
        v = valid[r0:r1]
        y = np.where(v, labels[r0:r1], 0)
        z_y = Zp[np.arange(r1 - r0), y]
        lse[r0:r1] = l
        zt[r0:r1] = np.where(v, z_y, 0.0)
        tok[r0:r1] = np.where(v, l - z_y, 0.0)
    return lse, tok, zt


def logits_rows(h: np.ndarray, W: np.ndarray, softcap: float) -> np.ndarray:
    """The logits Z' = softcap(h @ W.T) of every row of h, in float64.

    What a caller that needs the logits gets back (LlamaFactory error page,
    "Source" and "Solutions": with require_logits the logits must exist, which
    the plain cross-entropy path provides); the same Z' the loss is formed from.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    Zp, _ = softcap_logits(h @ W.T, softcap)
    return Zp


def grad_logits_rows(Zp: np.ndarray, dcap: Optional[np.ndarray], lse: np.ndarray,
                     labels: np.ndarray, valid: np.ndarray, c: float) -> np.ndarray:
    """dLoss/dZ for a block of rows: c * valid * (softmax(Z') - onehot(y)) * dZ'/dZ."""
    P = np.exp(Zp - lse[:, None])
    rows = np.flatnonzero(valid)
    P[rows, labels[rows]] -= 1.0
    G = P * (c * valid.astype(np.float64))[:, None]
    if dcap is not None:
        G = G * dcap
    return G


def flce_reference(h, W, labels, *, ignore_index: int = -100, softcap: float = 0.0,
                   reduction: str = "sum", num_label_tokens: Optional[int] = None,
                   mb_scale: float = 1.0, row_chunk: int = 1024) -> OracleResult:
    """Loss, num_tokens, dH and dW of fused linear cross-entropy, in float64.

    h: [N, H], W: [V, H], labels: [N] int. Values are widened exactly to float64.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64).reshape(-1)
    N, H = h.shape
    V = W.shape[0]
    if W.shape[1] != H or labels.shape[0] != N:
        raise ValueError("shape mismatch")
    valid = valid_mask(labels, ignore_index)
    check_labels(labels, valid, V)
    n = count_valid(valid)
    c = scale_factor(n, reduction, num_label_tokens, mb_scale)

    lse = np.zeros(N)
    tok = np.zeros(N)
    dH = np.zeros((N, H))
    dW = np.zeros((V, H))
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        hc = h[r0:r1]
        Zp, dcap = softcap_logits(hc @ W.T, softcap)
        l = logsumexp_rows(Zp)
        v = valid[r0:r1]
        y = np.where(v, labels[r0:r1], 0)
        z_y = Zp[np.arange(r1 - r0), y]
        lse[r0:r1] = l
        tok[r0:r1] = np.where(v, l - z_y, 0.0)
        G = grad_logits_rows(Zp, dcap, l, y, v, c)
        dH[r0:r1] = G @ W
        dW += G.T @ hc
    S = math.fsum(tok.tolist())
    loss64 = c * S
    return OracleResult(
        loss64=loss64, loss32=float(np.float32(loss64)),
        num_tokens=num_tokens_for(n, reduction), n_valid=n, c=c,
        dH=dH, dW=dW, lse=lse, token_loss=tok,
    )


def dW_rows(h, W, labels, lse, vocab_rows, *, c: float, ignore_index: int = -100,
            softcap: float = 0.0) -> np.ndarray:
    """dW[v, :] for selected vocabulary rows, given the per-token lse of all tokens.

    dW[v] = sum_i G[i, v] h_i with G[i, v] = c*valid_i*(exp(Z'_iv - lse_i) - [y_i = v])
    * dZ'/dZ -- only column v of the logits is needed, so full-size cases can be
    checked on sampled rows.
    """
    h = np.asarray(h, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels = np.asarray(labels, dtype=np.int64).reshape(-1)
    valid = valid_mask(labels, ignore_index)
    vocab_rows = np.asarray(vocab_rows, dtype=np.int64)
    Zc = h @ W[vocab_rows].T                       # [N, k]
    Zp, dcap = softcap_logits(Zc, softcap)
    P = np.exp(Zp - np.asarray(lse, dtype=np.float64)[:, None])
    onehot = (labels[:, None] == vocab_rows[None, :]) & valid[:, None]
    G = (P - onehot) * (c * valid.astype(np.float64))[:, None]
    if dcap is not None:
        G = G * dcap
    return G.T @ h


def dH_rows(h_rows, W, labels_rows, lse_rows, *, c: float, ignore_index: int = -100,
            softcap: float = 0.0) -> np.ndarray:
    """dH for selected tokens: dH_i = sum_v G[i, v] W_v, with G from the token's own
    logits row and its lse (only the token's row of the logits is needed)."""
    h_rows = np.asarray(h_rows, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    labels_rows = np.asarray(labels_rows, dtype=np.int64).reshape(-1)
    valid = valid_mask(labels_rows, ignore_index)
    Zp, dcap = softcap_logits(h_rows @ W.T, softcap)
    y = np.where(valid, labels_rows, 0)
    G = grad_logits_rows(Zp, dcap, np.asarray(lse_rows, dtype=np.float64), y, valid, c)
    return G @ W


def micro_batch_scale(n_mb: int, n_total: int, reduction: str) -> float:
    """Token-weighted micro-batch scale: 1.0 for 'sum'; n_mb / n_total for 'mean'.

    twinkle PR 335, "PR information", item 2 (same token-weighted scale as the
    plain cross-entropy loss, 1.0 for 'sum'); with it the micro-batch means add
    up to the mean over the whole batch.
    """
    if reduction == "sum":
        return 1.0
    if reduction == "mean":
        return n_mb / n_total if n_total > 0 else 0.0
    raise ValueError(reduction)
