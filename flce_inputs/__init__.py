"""Seeded synthetic inputs for fused linear cross-entropy.

This module only draws random tensors and places ignore markers. It holds none
of the loss arithmetic, so both the float64 oracle (through the tests) and the
GPU path can be fed the exact same values.

Workload recipe (shapes and distributions from the five configurations this
library is measured on):

* hidden states ``h`` ~ N(0, 1), weight ``W`` ~ N(0, std) with std 0.02
  (0.03 for the softcapped case); drawn in float32 with ``torch.randn`` and a
  seeded CPU generator, then rounded to bfloat16 (round-to-nearest-even) for
  the bf16 cases.
* labels uniform in [0, V), or a Zipf(1.1) law truncated to V ranks (rank r has
  probability proportional to r**-1.1, token id r-1), drawn by inverse CDF
  from a seeded uniform.
* ignored positions: exactly floor(p*N) positions chosen by a seeded
  permutation ("p% ignored"), the first quarter of every sequence (masked
  prompt), or one contiguous span of flattened tokens.
* seeds: configuration k uses 1000*k + {0: h, 1: W, 2: labels, 3: mask}.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

IGNORE_INDEX = -100

__all__ = [
    "IGNORE_INDEX",
    "Workload",
    "RECIPES",
    "make_workload",
    "make_labels",
    "make_custom",
    "zipf_labels",
]


@dataclasses.dataclass
class Workload:
    name: str
    h: torch.Tensor            # [B, S, H] float32 or bfloat16, CPU
    W: torch.Tensor            # [V, H]
    labels: torch.Tensor       # [B, S] int64
    ignore_index: int
    softcap: float
    reduction: str
    num_label_tokens: Optional[int]
    micro_batches: int
    expected_valid: int        # count fixed by construction
    std_w: float

    @property
    def N(self) -> int:
        return self.h.shape[0] * self.h.shape[1]

    @property
    def H(self) -> int:
        return self.h.shape[-1]

    @property
    def V(self) -> int:
        return self.W.shape[0]

    @property
    def dtype(self) -> torch.dtype:
        return self.h.dtype


# name, B, S, H, V, dtype, w_std, label law, mask law, softcap, reduction, T, micro-batches
RECIPES = {
    1: dict(name="tiny", B=2, S=16, H=64, V=1024, dtype=torch.float32, w_std=0.02,
            labels="uniform", mask=("frac", 0.10), softcap=0.0, reduction="sum",
            T=None, mb=1),
    2: dict(name="small", B=4, S=512, H=1024, V=32000, dtype=torch.bfloat16, w_std=0.02,
            labels="uniform", mask=("frac", 0.05), softcap=0.0, reduction="sum",
            T=None, mb=1),
    3: dict(name="large_vocab", B=2, S=4096, H=4096, V=131072, dtype=torch.bfloat16,
            w_std=0.02, labels="zipf", mask=("prefix", 0.25), softcap=0.0,
            reduction="mean", T=None, mb=1),
    4: dict(name="softcapped", B=2, S=4096, H=3584, V=256000, dtype=torch.bfloat16,
            w_std=0.03, labels="uniform", mask=("frac", 0.10), softcap=30.0,
            reduction="sum", T=None, mb=1),
    5: dict(name="long_edge", B=2, S=8192, H=4096, V=131072, dtype=torch.bfloat16,
            w_std=0.02, labels="uniform", mask=("span", 7936, 8448), softcap=0.0,
            reduction="sum", T=15872, mb=4),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def _randn(shape, std: float, seed: int, dtype: torch.dtype, chunk_rows: int = 16384):
    """N(0, std) drawn in float32 from one seeded stream, then rounded to dtype.

    Rows are drawn in fixed chunks of ``chunk_rows`` from one generator, so the
    peak host memory of a [256000, 3584] draw stays near one float32 chunk. The
    chunking is part of the definition of the stream (the same call always gives
    the same values).
    """
    g = _gen(seed)
    rows = shape[0]
    rest = tuple(shape[1:])
    out = torch.empty((rows,) + rest, dtype=dtype)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = torch.randn((r1 - r0,) + rest, generator=g, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[r0:r1] = x.to(dtype)
    return out


def zipf_labels(n: int, V: int, s: float, seed: int) -> torch.Tensor:
    """Truncated Zipf(s) over V ranks by inverse CDF; token id = rank - 1."""
    g = _gen(seed)
    ranks = torch.arange(1, V + 1, dtype=torch.float64)
    w = ranks.pow(-s)
    cdf = torch.cumsum(w, 0)
    cdf = cdf / cdf[-1]
    u = torch.rand(n, generator=g, dtype=torch.float64)
    idx = torch.searchsorted(cdf, u, right=False)
    return idx.clamp_(0, V - 1).to(torch.int64)


def _uniform_labels(n: int, V: int, seed: int) -> torch.Tensor:
    return torch.randint(0, V, (n,), generator=_gen(seed), dtype=torch.int64)


def _apply_mask(labels: torch.Tensor, B: int, S: int, mask, seed: int,
                ignore_index: int) -> int:
    """Place ignore markers in the flattened labels in place; returns the count."""
    n = labels.numel()
    kind = mask[0]
    if kind == "frac":
        k = int(math.floor(mask[1] * n))
        pos = torch.randperm(n, generator=_gen(seed))[:k]
        labels[pos] = ignore_index
        return k
    if kind == "prefix":
        q = int(S * mask[1])
        lab = labels.view(B, S)
        lab[:, :q] = ignore_index
        return B * q
    if kind == "span":
        a, b = mask[1], mask[2]
        labels[a:b] = ignore_index
        return b - a
    if kind == "none":
        return 0
    raise ValueError(f"unknown mask {mask!r}")


def make_labels(k: int, *, scale_tokens: Optional[int] = None):
    """Labels [N] (int64) of configuration k and the number of ignored positions."""
    c = RECIPES[k]
    B, S, V = c["B"], c["S"], c["V"]
    if scale_tokens is not None:
        S = scale_tokens
    base = 1000 * k
    N = B * S
    if c["labels"] == "uniform":
        labels = _uniform_labels(N, V, base + 2)
    else:
        labels = zipf_labels(N, V, 1.1, base + 2)
    mask = c["mask"]
    if mask[0] == "span" and scale_tokens is not None:
        mask = ("span", min(mask[1], N), min(mask[2], N))
    ignored = _apply_mask(labels, B, S, mask, base + 3, IGNORE_INDEX)
    return labels, ignored


def make_workload(k: int, *, scale_tokens: Optional[int] = None) -> Workload:
    """Build configuration k (1..5) exactly as specified, on the CPU.

    ``scale_tokens`` (optional) keeps everything but draws only the first
    ``scale_tokens`` sequence positions of each sequence -- never used for the
    measured workload, only to make a smaller case with the same recipe.
    """
    c = RECIPES[k]
    B, S, H, V = c["B"], c["S"], c["H"], c["V"]
    if scale_tokens is not None:
        S = scale_tokens
    base = 1000 * k
    N = B * S
    labels, ignored = make_labels(k, scale_tokens=scale_tokens)
    h = _randn((N, H), 1.0, base + 0, c["dtype"]).view(B, S, H)
    W = _randn((V, H), c["w_std"], base + 1, c["dtype"])
    return Workload(
        name=c["name"], h=h, W=W, labels=labels.view(B, S), ignore_index=IGNORE_INDEX,
        softcap=c["softcap"], reduction=c["reduction"], num_label_tokens=c["T"],
        micro_batches=c["mb"], expected_valid=N - ignored, std_w=c["w_std"],
    )


def make_custom(N: int, H: int, V: int, *, dtype=torch.bfloat16, seed: int = 7,
                w_std: float = 0.02, h_std: float = 1.0, ignore_frac: float = 0.1,
                labels: str = "uniform", softcap: float = 0.0,
                reduction: str = "sum", num_label_tokens: Optional[int] = None,
                ignore_index: int = IGNORE_INDEX) -> Workload:
    """A seeded case of any shape with the same recipe (B=1, S=N)."""
    h = _randn((N, H), h_std, seed * 10 + 0, dtype) if N > 0 else torch.empty(N, H, dtype=dtype)
    W = _randn((V, H), w_std, seed * 10 + 1, dtype)
    if labels == "uniform":
        lab = _uniform_labels(N, V, seed * 10 + 2)
    elif labels == "zipf":
        lab = zipf_labels(N, V, 1.1, seed * 10 + 2)
    else:
        raise ValueError(labels)
    ignored = _apply_mask(lab, 1, N, ("frac", ignore_frac), seed * 10 + 3, ignore_index) if N else 0
    return Workload(
        name=f"custom_N{N}_H{H}_V{V}", h=h.view(1, N, H), W=W, labels=lab.view(1, N),
        ignore_index=ignore_index, softcap=softcap, reduction=reduction,
        num_label_tokens=num_label_tokens, micro_batches=1,
        expected_valid=N - ignored, std_w=w_std,
    )
