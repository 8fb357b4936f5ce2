"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare within the stated tolerances.

Tolerances on o (max-abs, float64 comparison): 2e-2 for bfloat16, 5e-3 for
float16, 1e-5 for float32.  On lse (natural-log log-sum-exp): 1e-4 for the
16-bit types and 1e-5 for float32; the 16-bit bound is looser than the
float32 one only because the scores come from rounded inputs feeding a
float32 accumulator, whose relative error (~1e-6) is far below it.
"""

from __future__ import annotations

import numpy as np
import torch

import scaled_dot_product_fwd_amd as sdpa
from oracle import sdpa_ref, sdpa_ref_rows
from scaled_dot_product_fwd_amd.synth import DTYPES, default_scale, make_qkv

TOL_O = {torch.float32: 1e-5, torch.float16: 5e-3, torch.bfloat16: 2e-2}
TOL_LSE = {torch.float32: 1e-5, torch.float16: 1e-4, torch.bfloat16: 1e-4}


def to_dtype(name):
    return DTYPES[name] if isinstance(name, str) else name


def run_gpu(q, k, v, scale, mask, window, poison=True, attn_mask=None, **plan):
    """Copy CPU inputs to cuda:0, run the fused forward, return CPU float64 (o, lse).

    ``attn_mask`` (a CPU mask array) goes to the device in the padded-row
    layout the library reads.
    """
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if attn_mask is not None:
        plan["attn_mask"] = sdpa.pad_mask(attn_mask.to(dev))
    b, hq, lq, _ = q.shape
    out = torch.empty((b, hq, lq, v.shape[3]), dtype=q.dtype, device=dev)
    lse = torch.empty((b, hq, lq), dtype=torch.float32, device=dev)
    if poison:  # any element the kernels fail to write stays NaN
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
    o, l = sdpa.forward(qd, kd, vd, scale=scale, mask=mask, window_size=window, return_lse=True,
                        out=out, lse_out=lse, **plan)
    torch.cuda.synchronize()
    return o.cpu().to(torch.float64).numpy(), l.cpu().to(torch.float64).numpy()


def lse_err(got, ref):
    """max |got - ref| where equal infinities (rows with no kept key) count as 0."""
    same_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(got - ref))
    return float(d.max()) if d.size else 0.0


def check_full(b, hq, hkv, lq, lk, dqk, dv, dtype, mask="none", window=0, seed=0, scale=None,
               attn_mask=None, **plan):
    """Element-by-element parity of the whole output against the oracle.

    ``attn_mask`` is an optional CPU mask array (bool or the input dtype)
    broadcastable to [b, hq, lq, lk].
    """
    dt = to_dtype(dtype)
    q, k, v = make_qkv(b, hq, hkv, lq, lk, dqk, dv, dt, seed)
    scale = default_scale(dqk) if scale is None else scale
    o, lse = run_gpu(q, k, v, scale, mask, window, attn_mask=attn_mask, **plan)
    ro, rl = sdpa_ref(q, k, v, scale, mask, window, mask_arr=attn_mask)
    assert not np.isnan(o).any(), "unwritten (NaN) output elements"
    assert not np.isnan(lse).any(), "unwritten (NaN) lse elements"
    eo = float(np.abs(o - ro).max())
    el = lse_err(lse, rl)
    assert eo <= TOL_O[dt], f"max|o - ref| = {eo:.3e} > {TOL_O[dt]:.0e}"
    assert el <= TOL_LSE[dt], f"max|lse - ref| = {el:.3e} > {TOL_LSE[dt]:.0e}"
    return eo, el


def pick_rows(b, hq, lq, n, seed, window=0):
    """Sampled (b, h, i) rows: random ones plus the first/last rows and window edges."""
    rng = np.random.default_rng(seed)
    n = min(n, b * hq * lq)  # never ask for more distinct rows than exist
    rows = {(0, 0, 0), (b - 1, hq - 1, lq - 1), (0, hq - 1, lq // 2)}
    for i in (1, 2, 63, 64, 65, 127, 128, window - 1, window, window + 1, lq - 2):
        if 0 <= i < lq:
            rows.add((int(rng.integers(b)), int(rng.integers(hq)), i))
    while len(rows) < n:
        rows.add((int(rng.integers(b)), int(rng.integers(hq)), int(rng.integers(lq))))
    return sorted(rows)


def check_sampled(b, hq, hkv, lq, lk, dqk, dv, dtype, mask="none", window=0, seed=0, nrows=48,
                  attn_mask=None, **plan):
    """Full-size run on the GPU; the oracle recomputes sampled rows one by one."""
    dt = to_dtype(dtype)
    q, k, v = make_qkv(b, hq, hkv, lq, lk, dqk, dv, dt, seed)
    scale = default_scale(dqk)
    o, lse = run_gpu(q, k, v, scale, mask, window, attn_mask=attn_mask, **plan)
    assert not np.isnan(o).any(), "unwritten (NaN) output elements"
    assert not np.isnan(lse).any(), "unwritten (NaN) lse elements"
    picks = pick_rows(b, hq, lq, nrows, seed + 7, window)
    ro, rl = sdpa_ref_rows(q, k, v, scale, mask, window, picks, mask_arr=attn_mask)
    go = np.stack([o[p] for p in picks])
    gl = np.array([lse[p] for p in picks])
    eo = float(np.abs(go - ro).max())
    el = lse_err(gl, rl)
    assert eo <= TOL_O[dt], f"max|o - ref| = {eo:.3e} > {TOL_O[dt]:.0e} on sampled rows"
    assert el <= TOL_LSE[dt], f"max|lse - ref| = {el:.3e} > {TOL_LSE[dt]:.0e} on sampled rows"
    return eo, el
