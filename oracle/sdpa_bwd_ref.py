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

from .sdpa_ref import _as_f64, _dims, _lens, visible_mask, visible_offset


def sdpa_bwd_ref(q, k, v, do, scale: float, mask: str = "none", window: int = 0):
    """Returns ``(dq, dk, dv)`` in float64 with the shapes of q, k, v."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    b, hq, hkv, lq, lk, dqk, dv_ = _dims(q, k, v)
    if do.shape != (b, hq, lq, dv_):
        raise ValueError("do must be [B, Hq, Lq, Dv]")
    vis = visible_mask(lq, lk, mask, window)
    group = hq // hkv
    scale = float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(b):
        for h in range(hq):
            kvh = h // group
            s = np.where(vis, scale * (q[bi, h] @ k[bi, kvh].T), -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dv[bi, kvh] += p.T @ do[bi, h]
            dp = do[bi, h] @ v[bi, kvh].T
            d = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - d)
            dq[bi, h] = scale * (ds @ k[bi, kvh])
            dk[bi, kvh] += scale * (ds.T @ q[bi, h])
    return dq, dk, dv


def sdpa_bwd_ref_varlen(q, k, v, do, scale: float, mask: str = "none", window: int = 0, q_lens=None,
                        kv_lens=None):
    """Gradients with per-batch lengths, as ``(dq, dk, dv)`` in float64 with
    the padded shapes.  Entry b uses its first ``q_lens[b]`` queries and
    ``kv_lens[b]`` keys, query i at key position ``i + kv_lens[b] - q_lens[b]``
    (the forward's reading); the outputs past the lengths do not depend on any
    input, so every gradient position past them is 0, and so is a row that
    sees no key (its output is the constant 0)."""
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    b, hq, hkv, lq, lk, dqk, dv_ = _dims(q, k, v)
    if do.shape != (b, hq, lq, dv_):
        raise ValueError("do must be [B, Hq, Lq, Dv]")
    ql = _lens(q_lens, b, lq, "q_lens")
    kl = _lens(kv_lens, b, lk, "kv_lens")
    group = hq // hkv
    scale = float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(b):
        nq, nk = int(ql[bi]), int(kl[bi])
        if nq == 0 or nk == 0:
            continue
        vis = visible_offset(nq, nk, nk - nq, mask, window)
        seen = vis.any(axis=1)  # rows with at least one key
        for h in range(hq):
            kvh = h // group
            s = np.where(vis, scale * (q[bi, h, :nq] @ k[bi, kvh, :nk].T), -np.inf)
            m = np.where(seen[:, None], s.max(axis=1, keepdims=True), 0.0)
            p = np.where(vis, np.exp(s - m), 0.0)
            den = p.sum(axis=1, keepdims=True)
            p = np.divide(p, den, out=np.zeros_like(p), where=den > 0)
            g = do[bi, h, :nq]
            dv[bi, kvh, :nk] += p.T @ g
            dp = g @ v[bi, kvh, :nk].T
            d = (p * dp).sum(axis=1, keepdims=True)
            ds = p * (dp - d)
            dq[bi, h, :nq] = scale * (ds @ k[bi, kvh, :nk])
            dk[bi, kvh, :nk] += scale * (ds.T @ q[bi, h, :nq])
    return dq, dk, dv
