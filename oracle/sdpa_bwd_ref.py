"""Plain float64 CPU definition of the scaled-dot-product attention backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

With ``S = scale * Q K^T`` (masked entries -inf), ``P = softmax(S)`` per row
and ``O = P V``, the gradients of a loss with upstream gradient ``dO`` are the
textbook ones of softmax attention:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij            (= dO_i . O_i)
    dS = P * (dP - D)                 (elementwise, D broadcast over keys)
    dQ = scale * dS K
    dK = scale * dS^T Q

Under grouped-query attention a KV head's dK and dV sum the contributions of
its G query heads.  The pages name the backward pass (VJP) as the training
workload outside the fused forward (mlx PR #4185 "Add force_fused option to
scaled_dot_product_attention", Background: training still takes the unfused
path; mlx PR #3552 "feat(fast): add sliding-window SDPA kernel path",
Outstanding: VJP support not extended), and the forward's log-sum-exp output
as what it needs (mlx PR #4185, API).  Visibility follows the forward oracle
(bottom-right causal, window).  Everything is float64 after an exact upcast.
"""

from __future__ import annotations

import numpy as np

from .sdpa_ref import _apply, _as_f64, _dims, _lens, _softmax_rows, mask_array, visible_mask, visible_offset


def _bwd_heads(q, k, v, do, scale, vis, arr, group, dq, dk, dv):
    """Accumulate the gradients of one batch entry (arrays ``[H, L, D]``):
    scores with the mode's visibility and the mask array applied, softmax
    per row (a row with no key left gets P = 0), then the textbook formulas."""
    for h in range(q.shape[0]):
        kvh = h // group
        s = _apply(scale * (q[h] @ k[kvh].T), vis, None if arr is None else arr[h])
        p, den, _, empty = _softmax_rows(s)
        p = np.where(empty, 0.0, p / np.where(empty, 1.0, den))
        dv[kvh] += p.T @ do[h]
        dp = do[h] @ v[kvh].T
        d = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - d)
        dq[h] = scale * (ds @ k[kvh])
        dk[kvh] += scale * (ds.T @ q[h])


def sdpa_bwd_ref(q, k, v, do, scale: float, mask: str = "none", window: int = 0, mask_arr=None):
    """Returns ``(dq, dk, dv)`` in float64 with the shapes of q, k, v.
    ``mask_arr`` (optional) is the forward's explicit mask array: boolean
    (True keeps a key) or additive (added to the scaled scores)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    b, hq, hkv, lq, lk, dqk, dv_ = _dims(q, k, v)
    if do.shape != (b, hq, lq, dv_):
        raise ValueError("do must be [B, Hq, Lq, Dv]")
    vis = visible_mask(lq, lk, mask, window)
    arr = mask_array(mask_arr, b, hq, lq, lk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(b):
        _bwd_heads(q[bi], k[bi], v[bi], do[bi], float(scale), vis, None if arr is None else arr[bi],
                   hq // hkv, dq[bi], dk[bi], dv[bi])
    return dq, dk, dv


def sdpa_bwd_ref_varlen(q, k, v, do, scale: float, mask: str = "none", window: int = 0, q_lens=None,
                        kv_lens=None, mask_arr=None):
    """Gradients with per-batch lengths, as ``(dq, dk, dv)`` in float64 with
    the padded shapes.  Entry b uses its first ``q_lens[b]`` queries and
    ``kv_lens[b]`` keys, query i at key position ``i + kv_lens[b] - q_lens[b]``
    (the forward's reading); the outputs past the lengths do not depend on any
    input, so every gradient position past them is 0, and so is a row that
    sees no key (its output is the constant 0).  ``mask_arr`` is indexed in
    the padded coordinates ``(b, h, i, j)``."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    b, hq, hkv, lq, lk, dqk, dv_ = _dims(q, k, v)
    if do.shape != (b, hq, lq, dv_):
        raise ValueError("do must be [B, Hq, Lq, Dv]")
    ql = _lens(q_lens, b, lq, "q_lens")
    kl = _lens(kv_lens, b, lk, "kv_lens")
    arr = mask_array(mask_arr, b, hq, lq, lk)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(b):
        nq, nk = int(ql[bi]), int(kl[bi])
        if nq == 0 or nk == 0:
            continue
        vis = visible_offset(nq, nk, nk - nq, mask, window)
        _bwd_heads(q[bi, :, :nq], k[bi, :, :nk], v[bi, :, :nk], do[bi, :, :nq], float(scale), vis,
                   None if arr is None else arr[bi, :, :nq, :nk], hq // hkv, dq[bi, :, :nq], dk[bi, :, :nk],
                   dv[bi, :, :nk])
    return dq, dk, dv
