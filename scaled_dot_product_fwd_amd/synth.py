"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds random-number plumbing only, none of the attention
arithmetic.  Inputs are drawn as N(0, 1) in float32 on the CPU from a
``torch.Generator`` seeded with ``seed`` (q), ``seed + 1`` (k) and
``seed + 2`` (v), then cast to the compute dtype (round to nearest even), so
the HIP path and the oracle read the very same values.  Layout is contiguous
``[B, H, L, D]``.
"""

from __future__ import annotations

from typing import Tuple

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def randn(shape, seed: int, dtype: torch.dtype) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(dtype).contiguous()


def make_qkv(b: int, hq: int, hkv: int, lq: int, lk: int, dqk: int, dv: int,
             dtype: torch.dtype, seed: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """CPU tensors q ``[b,hq,lq,dqk]``, k ``[b,hkv,lk,dqk]``, v ``[b,hkv,lk,dv]``."""
    q = randn((b, hq, lq, dqk), seed, dtype)
    k = randn((b, hkv, lk, dqk), seed + 1, dtype)
    v = randn((b, hkv, lk, dv), seed + 2, dtype)
    return q, k, v


def default_scale(dqk: int) -> float:
    """1/sqrt(Dqk) rounded to float32, the value handed to both sides."""
    return float(torch.tensor(dqk, dtype=torch.float64).rsqrt().to(torch.float32))


def bool_mask(shape, seed: int, keep: float) -> torch.Tensor:
    """CPU boolean mask array: each element True (key kept) with probability ``keep``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.rand(tuple(shape), generator=g, dtype=torch.float32) < keep


def additive_mask(shape, seed: int, dtype: torch.dtype, sigma: float = 2.0,
                  minus_inf: float = 0.2) -> torch.Tensor:
    """CPU additive mask array: N(0, sigma^2) values rounded to ``dtype``, and
    -inf with probability ``minus_inf``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    vals = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * sigma
    drop = torch.rand(tuple(shape), generator=g, dtype=torch.float32) < minus_inf
    return vals.masked_fill(drop, float("-inf")).to(dtype)


def lengths(n: int, lo: int, hi: int, seed: int) -> torch.Tensor:
    """CPU int32 ``[n]``: lengths drawn uniformly from [lo, hi]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randint(lo, hi + 1, (n,), generator=g).to(torch.int32)


def padding_mask(b: int, lk: int, seed: int, min_len: int = 1) -> torch.Tensor:
    """CPU key-padding mask ``[b, 1, 1, lk]``: batch row n keeps its first
    len_n keys, the lengths being ``lengths(b, min_len, lk, seed)``."""
    lens = lengths(b, min_len, lk, seed).to(torch.int64)
    return (torch.arange(lk)[None, :] < lens[:, None]).reshape(b, 1, 1, lk)
