"""Plain float64 CPU definition of scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What is computed
----------------
``O = softmax(scale * Q K^T + mask) V`` per batch and query head, with

* grouped-query attention: query head ``h`` reads key/value head
  ``h // (Hq // Hkv)``, i.e. consecutive query heads share one KV head
  (the grouping factor is Hq // Hkv query heads per KV head; mlx issue #3826
  "2.3-2.8x latency jump from L=8 to L=12 queries", first maintainer comment,
  item 1).  This is
  the same as repeating every KV head ``Hq // Hkv`` times in place.
* causal masking aligned bottom-right: query row ``i`` sits at key position
  ``p = i + (Lk - Lq)`` and sees keys ``j <= p`` (K-relative coordinates with
  ``qL_off = kL - qL``; mlx PR #3552 "feat(fast): add sliding-window SDPA
  kernel path", Implementation).  ``Lq > Lk`` with a causal mask is an error
  (mlx PR #4185 "Add force_fused option to scaled_dot_product_attention",
  Validation).
* sliding window: each query sees only the last ``window`` key positions up to
  and including its own, combined with causal masking, i.e. ``p - W < j <= p``
  (mlx PR #3552, Summary, and the per-element rule in Implementation that
  removes a key once the query's position exceeds it by W or more).  ``window >= 1`` is required.
* an optional explicit mask array broadcast over ``[B, Hq, Lq, Lk]`` (the
  ``mask_arr`` argument beside the mask mode in mlx PR #3552, Public API; the
  boolean and float mask specialisations listed in mlx PR #4185's validation
  comment).  Boolean: True keeps the key, False removes it.  Float: the value
  is added to the scaled score, ``scale * q.k + mask``, in natural-log units,
  so ``-inf`` removes the key.  It combines with the mask mode: a key counts
  only if the mode and the array both keep it.
* a row that keeps no key at all (possible only through a mask array) has
  output 0 and log-sum-exp ``-inf``: the limit of a row whose every score goes
  to ``-inf``, and what the log-sum-exp merge of partial results gives for an
  empty part.
* the log-sum-exp of the visible scaled scores, natural log, per query row
  (the output that training needs; mlx PR #4185, API).
* optional per-batch lengths (``sdpa_ref_varlen``): batch entry b uses its
  first ``q_lens[b]`` queries and first ``kv_lens[b]`` keys, and its query i
  sits at key position ``i + kv_lens[b] - q_lens[b]``, the K-relative
  coordinates of mlx PR #3552 (Implementation: ``qL_off = kL - qL``, which
  the page notes also serves chunked prefill over a rotated cache) applied to
  the valid part.  Rows past ``q_lens[b]`` are not part of the result.  A
  row with no visible key (``kv_lens[b] = 0``, or a causal row placed before
  the first key) has output 0 and log-sum-exp ``-inf``.

Everything is evaluated in float64 after an exact upcast of the inputs, with
the full score rows materialised, which is the unfused "matmul -> softmax ->
matmul" shape the fused kernels avoid (mlx PR #4185, Background).
"""

from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

MASK_KINDS = ("none", "causal", "window")


def _as_f64(x) -> np.ndarray:
    """Exact upcast of a numpy array or a CPU torch tensor to float64."""
    if hasattr(x, "detach"):  # torch tensor: float16/bfloat16/float32 -> float64 is exact
        x = x.detach().to("cpu")
        import torch  # local: the oracle does not otherwise need torch

        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _check_mask(lq: int, lk: int, mask: str, window: int) -> None:
    if mask not in MASK_KINDS:
        raise ValueError(f"unknown mask kind {mask!r}")
    if mask != "none" and lq > lk:
        raise ValueError("causal masking needs Lq <= Lk (queries align to the last Lq keys)")
    if mask == "window" and window < 1:
        raise ValueError("a sliding window needs window >= 1")


def visible_mask(lq: int, lk: int, mask: str = "none", window: int = 0) -> np.ndarray:
    """Boolean ``[lq, lk]`` visibility: True where query row i may attend key j."""
    _check_mask(lq, lk, mask, window)
    if mask == "none":
        return np.ones((lq, lk), dtype=bool)
    pos = np.arange(lq, dtype=np.int64)[:, None] + (lk - lq)  # absolute key position of row i
    key = np.arange(lk, dtype=np.int64)[None, :]
    vis = key <= pos
    if mask == "window":
        vis &= key > pos - window
    return vis


def _visible_row(i: int, lq: int, lk: int, mask: str, window: int) -> np.ndarray:
    """Visibility of one query row, the same rule as ``visible_mask`` row by row."""
    key = np.arange(lk, dtype=np.int64)
    if mask == "none":
        return np.ones(lk, dtype=bool)
    pos = i + (lk - lq)
    vis = key <= pos
    if mask == "window":
        vis &= key > pos - window
    return vis


def visible_offset(lq: int, lk: int, off: int, mask: str = "none", window: int = 0) -> np.ndarray:
    """Boolean ``[lq, lk]`` visibility when query row i sits at key position
    ``i + off`` (any integer offset; rows may see no key)."""
    if mask not in MASK_KINDS:
        raise ValueError(f"unknown mask kind {mask!r}")
    if mask == "window" and window < 1:
        raise ValueError("a sliding window needs window >= 1")
    if mask == "none":
        return np.ones((lq, lk), dtype=bool)
    pos = np.arange(lq, dtype=np.int64)[:, None] + off
    key = np.arange(lk, dtype=np.int64)[None, :]
    vis = key <= pos
    if mask == "window":
        vis &= key > pos - window
    return vis


def visible_pairs(lq: int, lk: int, mask: str = "none", window: int = 0) -> int:
    """Number of visible (query, key) pairs of one head (counted, not derived)."""
    return int(visible_mask(lq, lk, mask, window).sum())


def mask_array(mask_arr, b: int, hq: int, lq: int, lk: int):
    """The explicit mask broadcast to ``[b, hq, lq, lk]`` (numpy view), or None.

    Boolean arrays stay boolean; anything else is upcast exactly to float64
    and must hold no NaN and no ``+inf``.
    """
    if mask_arr is None:
        return None
    if hasattr(mask_arr, "detach"):
        import torch

        t = mask_arr.detach().to("cpu")
        arr = t.numpy() if t.dtype == torch.bool else t.to(torch.float64).numpy()
    else:
        arr = np.asarray(mask_arr)
    if arr.dtype != np.bool_:
        arr = arr.astype(np.float64)
        if np.isnan(arr).any() or np.isposinf(arr).any():
            raise ValueError("an additive mask holds finite values or -inf")
    if arr.ndim > 4:
        raise ValueError("a mask array has at most 4 dims")
    return np.broadcast_to(arr, (b, hq, lq, lk))


def _apply(s: np.ndarray, vis: np.ndarray, arr) -> np.ndarray:
    """Scores with removed keys at -inf: mode visibility, then the mask array."""
    if arr is None:
        return np.where(vis, s, -np.inf)
    if arr.dtype == np.bool_:
        return np.where(vis & arr, s, -np.inf)
    return np.where(vis, s + arr, -np.inf)


def _softmax_rows(s: np.ndarray):
    """Softmax weights, denominators and maxima of score rows with -inf holes.

    A row with no finite score gets weights 0, denominator 0 and max -inf.
    """
    m = s.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    p = np.exp(s - np.where(empty, 0.0, m))  # exp(-inf) = 0 on removed keys
    den = p.sum(axis=-1, keepdims=True)
    return p, den, m, empty


def _dims(q, k, v) -> Tuple[int, int, int, int, int, int, int]:
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, D]")
    b, hq, lq, dqk = q.shape
    bk, hkv, lk, dk = k.shape
    bv, hv, lv, dv = v.shape
    if bk != b or bv != b or hv != hkv or lv != lk or dk != dqk:
        raise ValueError("inconsistent q/k/v shapes")
    if hq % hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return b, hq, hkv, lq, lk, dqk, dv


def sdpa_ref(q, k, v, scale: float, mask: str = "none", window: int = 0, chunk: int = 512,
             mask_arr=None):
    """Reference forward.  Returns ``(o, lse)`` in float64.

    ``o`` is ``[B, Hq, Lq, Dv]``, ``lse`` is ``[B, Hq, Lq]``.  ``scale`` is
    used as given (pass the same float32 value the GPU receives).
    ``mask_arr`` is an optional boolean or additive array broadcastable to
    ``[B, Hq, Lq, Lk]``.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, hq, hkv, lq, lk, dqk, dv = _dims(q, k, v)
    vis = visible_mask(lq, lk, mask, window)
    arr = mask_array(mask_arr, b, hq, lq, lk)
    group = hq // hkv
    scale = float(scale)
    o = np.zeros((b, hq, lq, dv), dtype=np.float64)
    lse = np.zeros((b, hq, lq), dtype=np.float64)
    for bi in range(b):
        for h in range(hq):
            kvh = h // group
            kt = k[bi, kvh].T
            vv = v[bi, kvh]
            for r0 in range(0, lq, chunk):
                r1 = min(lq, r0 + chunk)
                s = scale * (q[bi, h, r0:r1] @ kt)  # [rows, Lk] scaled scores
                s = _apply(s, vis[r0:r1], None if arr is None else arr[bi, h, r0:r1])
                p, den, m, empty = _softmax_rows(s)
                with np.errstate(divide="ignore", invalid="ignore"):
                    o[bi, h, r0:r1] = np.where(empty, 0.0, (p @ vv) / den)
                    lse[bi, h, r0:r1] = np.where(empty, -np.inf, m + np.log(den))[:, 0]
    return o, lse


def _lens(lens, n: int, cap: int, name: str) -> np.ndarray:
    """Per-batch lengths as int64, all of them, or ``cap`` for each entry when absent."""
    if lens is None:
        return np.full(n, cap, dtype=np.int64)
    if hasattr(lens, "detach"):
        lens = lens.detach().to("cpu").numpy()
    out = np.asarray(lens, dtype=np.int64).reshape(-1)
    if out.shape[0] != n or (out < 0).any() or (out > cap).any():
        raise ValueError(f"{name} must hold {n} lengths in [0, {cap}]")
    return out


def sdpa_ref_varlen(q, k, v, scale: float, mask: str = "none", window: int = 0, q_lens=None,
                    kv_lens=None, mask_arr=None):
    """Reference forward with per-batch lengths.  Returns ``(o, lse)`` in
    float64 with the padded shapes; rows ``i >= q_lens[b]`` are NaN (they are
    not part of the result).  ``mask_arr`` is indexed in the padded
    coordinates ``(b, h, i, j)``."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, hq, hkv, lq, lk, dqk, dv = _dims(q, k, v)
    ql = _lens(q_lens, b, lq, "q_lens")
    kl = _lens(kv_lens, b, lk, "kv_lens")
    arr = mask_array(mask_arr, b, hq, lq, lk)
    group = hq // hkv
    o = np.full((b, hq, lq, dv), np.nan)
    lse = np.full((b, hq, lq), np.nan)
    for bi in range(b):
        nq, nk = int(ql[bi]), int(kl[bi])
        vis = visible_offset(nq, nk, nk - nq, mask, window)
        for h in range(hq):
            kvh = h // group
            s = float(scale) * (q[bi, h, :nq] @ k[bi, kvh, :nk].T)
            s = _apply(s, vis, None if arr is None else arr[bi, h, :nq, :nk])
            if nk == 0:
                o[bi, h, :nq] = 0.0
                lse[bi, h, :nq] = -np.inf
                continue
            p, den, m, empty = _softmax_rows(s)
            with np.errstate(divide="ignore", invalid="ignore"):
                o[bi, h, :nq] = np.where(empty, 0.0, (p @ v[bi, kvh, :nk]) / den)
                lse[bi, h, :nq] = np.where(empty, -np.inf, m + np.log(den))[:, 0]
    return o, lse


def sdpa_probs(q, k, scale: float, mask: str = "none", window: int = 0, mask_arr=None) -> np.ndarray:
    """Attention probabilities ``[B, Hq, Lq, Lk]`` (tiny shapes only; an empty row is all 0)."""
    q, k = _as_f64(q), _as_f64(k)
    b, hq, lq, _ = q.shape
    hkv, lk = k.shape[1], k.shape[2]
    vis = visible_mask(lq, lk, mask, window)
    arr = mask_array(mask_arr, b, hq, lq, lk)
    group = hq // hkv
    out = np.zeros((b, hq, lq, lk), dtype=np.float64)
    for bi in range(b):
        for h in range(hq):
            s = float(scale) * (q[bi, h] @ k[bi, h // group].T)
            s = _apply(s, vis, None if arr is None else arr[bi, h])
            p, den, _, empty = _softmax_rows(s)
            with np.errstate(divide="ignore", invalid="ignore"):
                out[bi, h] = np.where(empty, 0.0, p / den)
    return out


def sdpa_ref_rows(q, k, v, scale: float, mask: str, window: int,
                  picks: Iterable[Sequence[int]], mask_arr=None, q_lens=None, kv_lens=None):
    """Reference output for selected rows only, for full-size sampled checks.

    ``picks`` holds ``(b, h, i)`` triples.  Returns ``(o_rows [n, Dv],
    lse_rows [n])`` in float64, with the same definition as ``sdpa_ref``.
    ``q``, ``k`` and ``v`` may be torch CPU tensors; only the rows touched are
    upcast.  ``mask_arr`` (optional) broadcasts to ``[B, Hq, Lq, Lk]`` as in
    ``sdpa_ref``; only the picked rows of it are read.  ``q_lens`` /
    ``kv_lens`` (optional) give per-batch lengths as in ``sdpa_ref_varlen``;
    picked rows must lie below ``q_lens[b]``.
    """
    picks = [tuple(int(t) for t in p) for p in picks]
    b, hq, lq, _ = q.shape
    hkv, lk = k.shape[1], k.shape[2]
    dv = v.shape[3]
    varlen = q_lens is not None or kv_lens is not None
    if not varlen:
        _check_mask(lq, lk, mask, window)
    ql = _lens(q_lens, b, lq, "q_lens")
    kl = _lens(kv_lens, b, lk, "kv_lens")
    group = hq // hkv
    arr = _mask_rows_view(mask_arr, b, hq, lq, lk)
    o = np.zeros((len(picks), dv), dtype=np.float64)
    lse = np.zeros(len(picks), dtype=np.float64)
    cache = {}
    for n, (bi, h, i) in enumerate(picks):
        kvh = h // group
        if (bi, kvh) not in cache:
            cache = {(bi, kvh): (_as_f64(k[bi, kvh]), _as_f64(v[bi, kvh]))}
        kk, vv = cache[(bi, kvh)]
        if varlen:
            nq, nk = int(ql[bi]), int(kl[bi])
            if i >= nq:
                raise ValueError("a picked row lies past q_lens[b]")
            vis = np.zeros(lk, dtype=bool)
            vis[:nk] = visible_offset(1, nk, i + nk - nq, mask, window)[0]
        else:
            vis = _visible_row(i, lq, lk, mask, window)
        s = float(scale) * (kk @ _as_f64(q[bi, h, i]))
        s = _apply(s, vis, None if arr is None else arr(bi, h, i))
        keep = np.isfinite(s)
        if not keep.any():
            o[n], lse[n] = 0.0, -math.inf
            continue
        s = s[keep]
        m = s.max()
        p = np.exp(s - m)
        den = p.sum()
        o[n] = (p @ vv[keep]) / den
        lse[n] = m + math.log(den)
    return o, lse


def _mask_rows_view(mask_arr, b, hq, lq, lk):
    """Row accessor ``(b, h, i) -> mask row [lk]`` that upcasts one row at a time."""
    if mask_arr is None:
        return None
    if hasattr(mask_arr, "detach"):
        t = mask_arr.detach()
        while t.dim() < 4:
            t = t.unsqueeze(0)
        t = t.expand(b, hq, lq, lk)
        return lambda bi, h, i: mask_array(t[bi, h, i], 1, 1, 1, lk)[0, 0, 0]
    arr = mask_array(mask_arr, b, hq, lq, lk)
    return lambda bi, h, i: arr[bi, h, i]


def sdpa_loop(q, k, v, scale: float, mask: str = "none", window: int = 0, mask_arr=None,
              q_lens=None, kv_lens=None):
    """Second formulation in pure Python loops (tiny shapes only).

    Walks each query row over the explicit key index range it may see and
    forms the softmax from ``exp(s - max)`` sums with ``math.fsum``.  A mask
    array entry is looked up per key: a boolean False or an additive -inf drops
    the key, another additive value is added to its score.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    b, hq, hkv, lq, lk, dqk, dv = _dims(q, k, v)
    varlen = q_lens is not None or kv_lens is not None
    if not varlen:
        _check_mask(lq, lk, mask, window)
    ql = _lens(q_lens, b, lq, "q_lens")
    kl = _lens(kv_lens, b, lk, "kv_lens")
    arr = mask_array(mask_arr, b, hq, lq, lk)
    group = hq // hkv
    o = np.full((b, hq, lq, dv), np.nan) if varlen else np.zeros((b, hq, lq, dv))
    lse = np.full((b, hq, lq), np.nan) if varlen else np.zeros((b, hq, lq))
    for bi in range(b):
        nq, nk = int(ql[bi]), int(kl[bi])
        for h in range(hq):
            kvh = h // group
            for i in range(nq):
                pos = i + nk - nq
                if mask == "none":
                    lo, hi = 0, nk - 1
                elif mask == "causal":
                    lo, hi = 0, min(pos, nk - 1)
                else:
                    lo, hi = max(0, pos - window + 1), min(pos, nk - 1)
                keys, s = [], []
                for j in range(lo, hi + 1):
                    sj = float(scale) * math.fsum(q[bi, h, i, d] * k[bi, kvh, j, d] for d in range(dqk))
                    if arr is not None:
                        a = arr[bi, h, i, j]
                        if arr.dtype == np.bool_:
                            if not a:
                                continue
                        elif a == -math.inf:
                            continue
                        else:
                            sj += float(a)
                    keys.append(j)
                    s.append(sj)
                if not keys:
                    o[bi, h, i, :] = 0.0
                    lse[bi, h, i] = -math.inf
                    continue
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                den = math.fsum(w)
                for c in range(dv):
                    o[bi, h, i, c] = math.fsum(w[t] * v[bi, kvh, j, c] for t, j in enumerate(keys)) / den
                lse[bi, h, i] = mx + math.log(den)
    return o, lse
