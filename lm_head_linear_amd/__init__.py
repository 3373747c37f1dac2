"""Fused linear cross-entropy (LM head + token cross-entropy) for MI355X.

A thin binding over libflce.so: the functions below marshal arguments into the
C-ABI of the same name; every step of the computation runs in the library's
HIP kernels. PyTorch supplies device memory and the current stream.

Contracts (see include/flce.h):
* ``reduction='sum'`` returns ``num_tokens`` = number of non-ignored tokens and,
  when ``num_label_tokens`` T > 0 is given, the loss divided by T;
  ``reduction='mean'`` returns ``num_tokens = 0`` (twinkle PR 335, "PR
  information", item 1). Apply exactly one normalisation: a sum loss already
  divided by T must not be divided by ``num_tokens`` again.
* an empty target set gives loss 0 and zero gradients (Ling-3.1-flash
  discussion 7), the loss is float32 for bf16 inputs (Modalities PR 464), and
  the softcap ``s*tanh(z/s)`` is applied on every path (twinkle PR 335 item 3).
* ``grad_dtype=torch.float32`` with bf16 inputs returns float32 dH and dW (the
  logit gradient kept as a bf16 hi + lo pair), for callers that accumulate
  gradients over micro-batches in float32; it costs twice the dW/dH work.
* ``recompute=False`` (bf16) is the no-recompute variant: tokens in chunks of
  ``token_chunk`` whose probabilities are kept (bf16, relative to each vocabulary
  tile's max) instead of recomputing the logits, 3 GEMM passes instead of 4, at
  the cost of token_chunk x V x 2 bytes of workspace.
* The forward call computes dH and dW as well; ``backward`` only scales them by
  the incoming gradient, on the device (no host synchronisation). When no
  gradient is wanted (``torch.no_grad()``, or neither input requires one) the
  forward-only entry runs instead: the same loss at a quarter of the work.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib

__all__ = [
    "flce_workspace_size",
    "flce_workspace_size_ex",
    "flce_vocab_chunk_ex",
    "flce_check_args",
    "flce_check_args_ex",
    "flce_check_args_nr",
    "flce_forward_backward",
    "flce_forward_backward_ex",
    "flce_forward_backward_nr",
    "flce_workspace_size_nr",
    "flce_token_chunk_nr",
    "flce_forward",
    "flce_forward_workspace_size",
    "flce_forward_check_args",
    "flce_forward_logits",
    "flce_forward_logits_check_args",
    "flce_forward_noalloc",
    "flce_status_string",
    "flce_vocab_chunk",
    "flce_kept_chunks",
    "flce_profile_begin",
    "flce_profile_end",
    "flce_profile_query",
    "flce_profile_kinds",
    "flce_kernel_kind_name",
    "kernel_kinds",
    "fused_linear_cross_entropy",
    "FusedLinearCrossEntropy",
    "FLCEFunction",
    "micro_batch_scale",
    "FlceError",
]


class FlceError(RuntimeError):
    def __init__(self, code: int, where: str = ""):
        self.code = code
        super().__init__(f"{where}: {flce_status_string(code)}" if where else flce_status_string(code))


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return _lib.BF16
    if dt == torch.float32:
        return _lib.F32
    raise ValueError(f"unsupported dtype {dt}; use torch.bfloat16 or torch.float32")


def _red_code(reduction: str) -> int:
    if reduction == "sum":
        return _lib.SUM
    if reduction == "mean":
        return _lib.MEAN
    raise ValueError(f"reduction must be 'sum' or 'mean', got {reduction!r}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def flce_status_string(code: int) -> str:
    return _lib.load().flce_status_string(int(code)).decode()


def flce_workspace_size(N: int, H: int, V: int, dtype: torch.dtype,
                        grad_dtype: Optional[torch.dtype] = None) -> int:
    g = _dtype_code(grad_dtype if grad_dtype is not None else dtype)
    return int(_lib.load().flce_workspace_size_ex(N, H, V, _dtype_code(dtype), g))


def flce_forward_workspace_size(N: int, H: int, V: int, dtype: torch.dtype) -> int:
    return int(_lib.load().flce_forward_workspace_size(N, H, V, _dtype_code(dtype)))


def flce_workspace_size_nr(N: int, H: int, V: int, dtype: torch.dtype, token_chunk: int = 0) -> int:
    return int(_lib.load().flce_workspace_size_nr(N, H, V, _dtype_code(dtype), int(token_chunk)))


def flce_token_chunk_nr(N: int, H: int, V: int, dtype: torch.dtype, token_chunk: int = 0) -> int:
    return int(_lib.load().flce_token_chunk_nr(N, H, V, _dtype_code(dtype), int(token_chunk)))


def flce_vocab_chunk(N: int, H: int, V: int, dtype: torch.dtype,
                     grad_dtype: Optional[torch.dtype] = None) -> int:
    g = _dtype_code(grad_dtype if grad_dtype is not None else dtype)
    return int(_lib.load().flce_vocab_chunk_ex(N, H, V, _dtype_code(dtype), g))


def flce_kept_chunks(N: int, H: int, V: int, dtype: torch.dtype,
                     accumulate_dW: bool = False) -> int:
    """Vocabulary chunks of flce_forward_backward whose logits are not
    recomputed (the forward keeps their probabilities)."""
    return int(_lib.load().flce_kept_chunks(N, H, V, _dtype_code(dtype), int(bool(accumulate_dW))))


def flce_workspace_size_ex(N: int, H: int, V: int, dtype: torch.dtype,
                           grad_dtype: torch.dtype) -> int:
    """Workspace of the float32-gradient entry (grad_dtype float32 with bf16)."""
    return flce_workspace_size(N, H, V, dtype, grad_dtype)


def flce_vocab_chunk_ex(N: int, H: int, V: int, dtype: torch.dtype,
                        grad_dtype: torch.dtype) -> int:
    return flce_vocab_chunk(N, H, V, dtype, grad_dtype)


def _abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens,
              loss, num_tokens, dH, dW, stream, dtype, mb_scale, accumulate_dW, workspace,
              status, lse_out):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(h), _ptr(W), _ptr(labels), N, H, V, int(ignore_index), float(softcap),
            _red_code(reduction), int(num_label_tokens or 0), _ptr(loss), _ptr(num_tokens),
            _ptr(dH), _ptr(dW), stream, _dtype_code(dtype), float(mb_scale),
            1 if accumulate_dW else 0, _ptr(workspace), ws_bytes, _ptr(status), _ptr(lse_out))


def flce_check_args(h, W, labels, *, N, H, V, ignore_index=-100, softcap=0.0, reduction="sum",
                    num_label_tokens=None, loss=None, num_tokens=None, dH=None, dW=None,
                    dtype=torch.bfloat16, mb_scale=1.0, accumulate_dW=False, workspace=None,
                    status=None, lse_out=None, grad_dtype=None) -> int:
    """The library's synchronous checks (no GPU work); returns a status code."""
    args = _abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens,
                     loss, num_tokens, dH, dW, None, dtype, mb_scale, accumulate_dW, workspace,
                     status, lse_out)
    g = _dtype_code(grad_dtype if grad_dtype is not None else dtype)
    return int(_lib.load().flce_check_args_ex(*args, g))


def flce_check_args_ex(h, W, labels, *, grad_dtype, **kw) -> int:
    """flce_check_args with the gradients' dtype given explicitly."""
    return flce_check_args(h, W, labels, grad_dtype=grad_dtype, **kw)


def flce_check_args_nr(h, W, labels, *, N, H, V, ignore_index=-100, softcap=0.0,
                       reduction="sum", num_label_tokens=None, loss=None, num_tokens=None,
                       dH=None, dW=None, dtype=torch.bfloat16, mb_scale=1.0,
                       accumulate_dW=False, workspace=None, status=None, lse_out=None,
                       token_chunk=0) -> int:
    """The no-recompute entry's synchronous checks (no GPU work); a status code."""
    args = _abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens,
                     loss, num_tokens, dH, dW, None, dtype, mb_scale, accumulate_dW, workspace,
                     status, lse_out)
    return int(_lib.load().flce_check_args_nr(*args, int(token_chunk)))


def _fwd_abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens,
                  loss, num_tokens, stream, dtype, mb_scale, workspace, status, lse_out):
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(h), _ptr(W), _ptr(labels), N, H, V, int(ignore_index), float(softcap),
            _red_code(reduction), int(num_label_tokens or 0), _ptr(loss), _ptr(num_tokens),
            stream, _dtype_code(dtype), float(mb_scale), _ptr(workspace), ws_bytes,
            _ptr(status), _ptr(lse_out))


def flce_forward_check_args(h, W, labels, *, N, H, V, ignore_index=-100, softcap=0.0,
                            reduction="sum", num_label_tokens=None, loss=None, num_tokens=None,
                            dtype=torch.bfloat16, mb_scale=1.0, workspace=None, status=None,
                            lse_out=None) -> int:
    """The forward-only entry's synchronous checks (no GPU work); a status code."""
    args = _fwd_abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                         num_label_tokens, loss, num_tokens, None, dtype, mb_scale, workspace,
                         status, lse_out)
    return int(_lib.load().flce_forward_check_args(*args))


def flce_forward_logits_check_args(h, W, labels, *, N, H, V, logits, ld_logits=None,
                                   logits_dtype=torch.float32, ignore_index=-100, softcap=0.0,
                                   reduction="sum", num_label_tokens=None, loss=None,
                                   num_tokens=None, dtype=torch.bfloat16, mb_scale=1.0,
                                   workspace=None, status=None, lse_out=None) -> int:
    """The logits-returning forward entry's synchronous checks; a status code."""
    args = _fwd_abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                         num_label_tokens, loss, num_tokens, None, dtype, mb_scale, workspace,
                         status, lse_out)
    ld = V if ld_logits is None else int(ld_logits)
    return int(_lib.load().flce_forward_logits_check_args(*args, _ptr(logits), ld,
                                                          _dtype_code(logits_dtype)))


def _check_tensor(name, t, shape, dtype, device):
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def flce_forward_backward(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, *,
                          ignore_index: int = -100, softcap: float = 0.0,
                          reduction: str = "sum", num_label_tokens: Optional[int] = None,
                          mb_scale: float = 1.0, dH: Optional[torch.Tensor] = None,
                          dW: Optional[torch.Tensor] = None, accumulate_dW: bool = False,
                          workspace: Optional[torch.Tensor] = None,
                          lse_out: Optional[torch.Tensor] = None,
                          status: Optional[torch.Tensor] = None,
                          loss: Optional[torch.Tensor] = None,
                          num_tokens: Optional[torch.Tensor] = None,
                          grad_dtype: Optional[torch.dtype] = None,
                          recompute: bool = True, token_chunk: int = 0):
    """One fused forward + backward on the current stream.

    h [N,H], W [V,H] (bf16 or fp32, same dtype, contiguous, on one GPU), labels
    [N] int64. Returns (loss fp32 scalar, num_tokens int64 scalar, dH, dW) as
    device tensors; nothing is synchronised. Output/workspace tensors may be
    passed in to avoid allocation. dH and dW have ``grad_dtype`` (default: the
    input dtype; float32 with bf16 inputs is the float32-gradient mode).
    ``recompute=False`` selects the no-recompute variant (bf16 inputs and
    gradients) with token chunks of ``token_chunk`` (0: automatic).
    """
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError("h must be [N, H] and W [V, H]")
    N, H = h.shape
    V = W.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("flce_forward_backward runs on a GPU; tensors are on " + str(dev))
    _check_tensor("h", h, (N, H), W.dtype, dev)
    _check_tensor("W", W, (V, H), W.dtype, dev)
    _check_tensor("labels", labels, (N,), torch.int64, dev)
    gdt = W.dtype if grad_dtype is None else grad_dtype
    _dtype_code(gdt)
    if dH is None:
        dH = torch.empty(N, H, dtype=gdt, device=dev)
    if dW is None:
        if accumulate_dW:
            raise ValueError("accumulate_dW needs the dW tensor to add to")
        dW = torch.empty(V, H, dtype=gdt, device=dev)
    _check_tensor("dH", dH, (N, H), gdt, dev)
    _check_tensor("dW", dW, (V, H), gdt, dev)
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if num_tokens is None:
        num_tokens = torch.empty((), dtype=torch.int64, device=dev)
    if lse_out is not None:
        _check_tensor("lse_out", lse_out, (N,), torch.float32, dev)
    if status is not None:
        _check_tensor("status", status, (), torch.int32, dev)
    if not recompute:
        if gdt != W.dtype:
            raise ValueError("the no-recompute variant returns gradients in the input dtype")
        need = flce_workspace_size_nr(N, H, V, W.dtype, token_chunk)
    else:
        need = flce_workspace_size(N, H, V, W.dtype, gdt)
    if need == 0:
        raise FlceError(_lib.ERR_UNSUPPORTED if W.dtype == torch.float32 else _lib.ERR_ARG,
                        "flce_workspace_size")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = _abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction, num_label_tokens,
                     loss, num_tokens, dH, dW, stream, W.dtype, mb_scale, accumulate_dW,
                     workspace, status, lse_out)
    with torch.cuda.device(dev):
        if recompute:
            rc = _lib.load().flce_forward_backward_ex(*args, _dtype_code(gdt))
        else:
            rc = _lib.load().flce_forward_backward_nr(*args, int(token_chunk))
    if rc != _lib.OK:
        raise FlceError(rc, "flce_forward_backward")
    return loss, num_tokens, dH, dW


def flce_forward_backward_ex(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, *,
                             grad_dtype: torch.dtype, **kw):
    """flce_forward_backward with dH and dW of dtype ``grad_dtype`` (float32 with
    bf16 inputs: the float32-gradient mode)."""
    return flce_forward_backward(h, W, labels, grad_dtype=grad_dtype, **kw)


def flce_forward_backward_nr(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, *,
                             token_chunk: int = 0, **kw):
    """The no-recompute variant: flce_forward_backward(..., recompute=False)."""
    return flce_forward_backward(h, W, labels, recompute=False, token_chunk=token_chunk, **kw)


def flce_forward(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, *,
                 ignore_index: int = -100, softcap: float = 0.0, reduction: str = "sum",
                 num_label_tokens: Optional[int] = None, mb_scale: float = 1.0,
                 workspace: Optional[torch.Tensor] = None,
                 lse_out: Optional[torch.Tensor] = None,
                 status: Optional[torch.Tensor] = None,
                 loss: Optional[torch.Tensor] = None,
                 num_tokens: Optional[torch.Tensor] = None):
    """Forward only (no gradients) on the current stream: (loss, num_tokens).

    Same inputs and contracts as :func:`flce_forward_backward`; the loss,
    count, lse and status are bit-identical to that call's.
    """
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError("h must be [N, H] and W [V, H]")
    N, H = h.shape
    V = W.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("flce_forward runs on a GPU; tensors are on " + str(dev))
    _check_tensor("h", h, (N, H), W.dtype, dev)
    _check_tensor("W", W, (V, H), W.dtype, dev)
    _check_tensor("labels", labels, (N,), torch.int64, dev)
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if num_tokens is None:
        num_tokens = torch.empty((), dtype=torch.int64, device=dev)
    if lse_out is not None:
        _check_tensor("lse_out", lse_out, (N,), torch.float32, dev)
    if status is not None:
        _check_tensor("status", status, (), torch.int32, dev)
    need = flce_forward_workspace_size(N, H, V, W.dtype)
    if need == 0:
        raise FlceError(_lib.ERR_ARG, "flce_forward_workspace_size")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = _fwd_abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                         num_label_tokens, loss, num_tokens, stream, W.dtype, mb_scale,
                         workspace, status, lse_out)
    with torch.cuda.device(dev):
        rc = _lib.load().flce_forward(*args)
    if rc != _lib.OK:
        raise FlceError(rc, "flce_forward")
    return loss, num_tokens


def flce_forward_noalloc(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, *,
                         ignore_index: int = -100, softcap: float = 0.0, reduction: str = "sum",
                         num_label_tokens: Optional[int] = None, mb_scale: float = 1.0,
                         loss: torch.Tensor, num_tokens: torch.Tensor,
                         lse_out: Optional[torch.Tensor] = None,
                         status: Optional[torch.Tensor] = None):
    """:func:`flce_forward` on the library's fixed per-GPU scratch (no workspace):
    the library allocates nothing, and this binding allocates nothing either, so
    the caller passes the output tensors. Problems whose forward workspace
    exceeds the scratch are refused (FlceError, FLCE_ERR_SCRATCH); overlapping
    calls on one GPU race on the shared scratch."""
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError("h must be [N, H] and W [V, H]")
    N, H = h.shape
    V = W.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("flce_forward_noalloc runs on a GPU; tensors are on " + str(dev))
    _check_tensor("h", h, (N, H), W.dtype, dev)
    _check_tensor("W", W, (V, H), W.dtype, dev)
    _check_tensor("labels", labels, (N,), torch.int64, dev)
    _check_tensor("loss", loss, (), torch.float32, dev)
    _check_tensor("num_tokens", num_tokens, (), torch.int64, dev)
    if lse_out is not None:
        _check_tensor("lse_out", lse_out, (N,), torch.float32, dev)
    if status is not None:
        _check_tensor("status", status, (), torch.int32, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = _lib.load().flce_forward_noalloc(
            _ptr(h), _ptr(W), _ptr(labels), N, H, V, int(ignore_index), float(softcap),
            _red_code(reduction), int(num_label_tokens or 0), _ptr(loss), _ptr(num_tokens),
            stream, _dtype_code(W.dtype), float(mb_scale), _ptr(status), _ptr(lse_out))
    if rc != _lib.OK:
        raise FlceError(rc, "flce_forward_noalloc")
    return loss, num_tokens


def flce_forward_logits(h: torch.Tensor, W: torch.Tensor, labels: torch.Tensor, *,
                        ignore_index: int = -100, softcap: float = 0.0, reduction: str = "sum",
                        num_label_tokens: Optional[int] = None, mb_scale: float = 1.0,
                        logits: Optional[torch.Tensor] = None,
                        logits_dtype: torch.dtype = torch.float32,
                        workspace: Optional[torch.Tensor] = None,
                        lse_out: Optional[torch.Tensor] = None,
                        status: Optional[torch.Tensor] = None,
                        loss: Optional[torch.Tensor] = None,
                        num_tokens: Optional[torch.Tensor] = None):
    """Forward that also returns the logits: (loss, num_tokens, logits).

    ``logits`` is [N, V] (or a row-strided view [N, V] of a wider buffer,
    unit stride along V), float32 or bfloat16: the softcapped logits the loss
    is formed from. A new contiguous [N, V] tensor of ``logits_dtype`` is made
    when it is None. Loss, count, lse and status are bit-identical to
    :func:`flce_forward`'s.
    """
    if h.dim() != 2 or W.dim() != 2:
        raise ValueError("h must be [N, H] and W [V, H]")
    N, H = h.shape
    V = W.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("flce_forward_logits runs on a GPU; tensors are on " + str(dev))
    _check_tensor("h", h, (N, H), W.dtype, dev)
    _check_tensor("W", W, (V, H), W.dtype, dev)
    _check_tensor("labels", labels, (N,), torch.int64, dev)
    if logits is None:
        logits = torch.empty((N, V), dtype=logits_dtype, device=dev)
    if logits.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    if tuple(logits.shape) != (N, V) or logits.device != dev:
        raise ValueError(f"logits must be [{N}, {V}] on {dev}")
    if N > 0 and V > 1 and logits.stride(1) != 1:
        raise ValueError("logits must have unit stride along the vocabulary")
    ld = logits.stride(0) if N > 1 else V
    if loss is None:
        loss = torch.empty((), dtype=torch.float32, device=dev)
    if num_tokens is None:
        num_tokens = torch.empty((), dtype=torch.int64, device=dev)
    if lse_out is not None:
        _check_tensor("lse_out", lse_out, (N,), torch.float32, dev)
    if status is not None:
        _check_tensor("status", status, (), torch.int32, dev)
    need = flce_forward_workspace_size(N, H, V, W.dtype)
    if need == 0:
        raise FlceError(_lib.ERR_ARG, "flce_forward_workspace_size")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = _fwd_abi_args(h, W, labels, N, H, V, ignore_index, softcap, reduction,
                         num_label_tokens, loss, num_tokens, stream, W.dtype, mb_scale,
                         workspace, status, lse_out)
    with torch.cuda.device(dev):
        rc = _lib.load().flce_forward_logits(*args, _ptr(logits), int(ld),
                                             _dtype_code(logits.dtype))
    if rc != _lib.OK:
        raise FlceError(rc, "flce_forward_logits")
    return loss, num_tokens, logits


def flce_profile_begin() -> None:
    _lib.load().flce_profile_begin()


def flce_profile_end() -> None:
    rc = _lib.load().flce_profile_end()
    if rc != _lib.OK:
        raise FlceError(rc, "flce_profile_end")


def flce_profile_kinds() -> int:
    return int(_lib.load().flce_profile_kinds())


def flce_kernel_kind_name(kind: int) -> str:
    return _lib.load().flce_kernel_kind_name(int(kind)).decode()


def kernel_kinds():
    return [flce_kernel_kind_name(k) for k in range(flce_profile_kinds())]


def flce_profile_query():
    """{kernel kind: (total ms, launches)} for the launches recorded since begin."""
    lib = _lib.load()
    out = {}
    for k in range(lib.flce_profile_kinds()):
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        rc = lib.flce_profile_query(k, ctypes.byref(ms), ctypes.byref(n))
        if rc != _lib.OK:
            raise FlceError(rc, "flce_profile_query")
        out[lib.flce_kernel_kind_name(k).decode()] = (ms.value, n.value)
    return out


def micro_batch_scale(n_mb: int, n_total: int, reduction: str) -> float:
    """Token-weighted micro-batch scale: 1.0 for 'sum', n_mb / n_total for 'mean'
    (twinkle PR 335, "PR information", item 2), so micro-batch losses add up to
    the loss of the whole batch."""
    if reduction == "sum":
        return 1.0
    if reduction == "mean":
        return float(n_mb) / float(n_total) if n_total > 0 else 0.0
    raise ValueError(reduction)


class FLCEFunction(torch.autograd.Function):
    """Autograd wrapper: the forward computes loss, dH and dW in one call."""

    @staticmethod
    def forward(ctx, h, W, labels, ignore_index, softcap, reduction, num_label_tokens, mb_scale):
        loss, num_tokens, dH, dW = flce_forward_backward(
            h.detach(), W.detach(), labels, ignore_index=ignore_index, softcap=softcap,
            reduction=reduction, num_label_tokens=num_label_tokens, mb_scale=mb_scale)
        ctx.save_for_backward(dH, dW)
        ctx.mark_non_differentiable(num_tokens)
        return loss, num_tokens

    @staticmethod
    def backward(ctx, grad_loss, grad_num_tokens):
        dH, dW = ctx.saved_tensors
        # d(g * loss) = g * (dH, dW), scaled on the device with no host sync:
        # the product is formed in float32 and rounded once to the gradient
        # dtype, so g == 1 returns dH and dW bit for bit and any other g adds
        # one rounding to the already rounded gradients.
        g = grad_loss.to(torch.float32)
        return torch.mul(dH, g), torch.mul(dW, g), None, None, None, None, None, None


def fused_linear_cross_entropy(hidden_states: torch.Tensor, labels: torch.Tensor,
                               lm_weight: torch.Tensor, *, ignore_index: int = -100,
                               softcap: float = 0.0, reduction: str = "sum",
                               num_label_tokens: Optional[int] = None, mb_scale: float = 1.0):
    """(loss, num_tokens) for hidden_states [..., H], labels [...], lm_weight [V, H]."""
    H = hidden_states.shape[-1]
    h = hidden_states.reshape(-1, H).contiguous()
    y = labels.reshape(-1).contiguous()
    if not (torch.is_grad_enabled() and (hidden_states.requires_grad or lm_weight.requires_grad)):
        return flce_forward(h.detach(), lm_weight.detach().contiguous(), y,
                            ignore_index=ignore_index, softcap=softcap, reduction=reduction,
                            num_label_tokens=num_label_tokens, mb_scale=mb_scale)
    return FLCEFunction.apply(h, lm_weight.contiguous(), y, ignore_index, softcap, reduction,
                              num_label_tokens, mb_scale)


class FusedLinearCrossEntropy(torch.nn.Module):
    """LM-head projection + cross-entropy without materialising logits.

    Same constructor and forward arguments as the fused module on the NeMo
    AutoModel linear_ce page (ignore_index=-100, logit_softcapping=0,
    reduction='sum'; forward(hidden_states [B,S,H], labels [B,S],
    lm_weight [V,H], num_label_tokens=None) -> scalar fp32 loss). After each
    call ``self.num_tokens`` holds the count contract of twinkle PR 335: the
    non-ignored token count for 'sum', 0 for 'mean'.
    """

    def __init__(self, ignore_index: int = -100, logit_softcapping: float = 0.0,
                 reduction: str = "sum"):
        super().__init__()
        if reduction not in ("sum", "mean"):
            raise ValueError(reduction)
        if logit_softcapping < 0:
            raise ValueError("logit_softcapping must be >= 0")
        self.ignore_index = ignore_index
        self.logit_softcapping = float(logit_softcapping)
        self.reduction = reduction
        self.num_tokens = None

    def forward(self, hidden_states, labels, lm_weight, num_label_tokens=None, mb_scale=1.0):
        loss, n = fused_linear_cross_entropy(
            hidden_states, labels, lm_weight, ignore_index=self.ignore_index,
            softcap=self.logit_softcapping, reduction=self.reduction,
            num_label_tokens=num_label_tokens, mb_scale=mb_scale)
        self.num_tokens = n
        return loss
