"""GPU parity of the backward pass (dQ, dK, dV) against the float64 oracle.

The forward runs on the GPU first (its o and lse feed the backward, as in
training); the oracle's gradients come from the definition alone.  Bound:
max |g - ref| <= TOL_REL * max |ref| per gradient, with TOL_REL = 1e-2 for
bfloat16 and 1.25e-3 for float16 -- two and a half units of the type's
rounding (u = 2^-8, 2^-11): P and dS are rounded to the input type before
their matrix products (one unit each, relative to the largest gradient
element) and each output once more, while the float32 accumulation adds far
less.  The cases below measure at most 1.3 units.
"""

import zlib

import numpy as np
import pytest
import torch

import scaled_dot_product_fwd_amd as sdpa
from oracle import sdpa_bwd_ref
from scaled_dot_product_fwd_amd.synth import default_scale, make_qkv, randn

pytestmark = pytest.mark.gpu

TOL_REL = {torch.bfloat16: 1e-2, torch.float16: 1.25e-3}


def _say(*a):
    print("CASE", *a, flush=True)


def run_bwd(b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, seed, scale=None, kv_parts=0):
    q, k, v = make_qkv(b, hq, hkv, lq, lk, dqk, dv, dt, seed)
    do = randn((b, hq, lq, dv), seed + 3, dt)
    scale = default_scale(dqk) if scale is None else scale
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    o, lse = sdpa.forward(qd, kd, vd, scale=scale, mask=mask, window_size=w, return_lse=True)
    grads = [torch.full_like(x, float("nan")) for x in (qd, kd, vd)]
    gq, gk, gv = sdpa.backward(qd, kd, vd, o, dod, lse, scale=scale, mask=mask, window_size=w,
                               dq=grads[0], dk=grads[1], dv=grads[2], kv_parts=kv_parts)
    torch.cuda.synchronize()
    ref = sdpa_bwd_ref(q, k, v, do, scale, mask, w)
    return [g.cpu().double().numpy() for g in (gq, gk, gv)], ref


def check_bwd(case, scale=None, kv_parts=0):
    b, hq, hkv, lq, lk, dqk, dv, dt, mask, w = case
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    got, ref = run_bwd(b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, zlib.crc32(repr(case).encode()) % 10000, scale,
                       kv_parts)
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert not np.isnan(g).any(), f"unwritten {name} elements"
        scale_ref = max(float(np.abs(r).max()), 1e-30)
        e = float(np.abs(g - r).max()) / scale_ref
        errs.append(e)
        assert e <= TOL_REL[dt], f"{name}: max|g - ref| / max|ref| = {e:.3e} > {TOL_REL[dt]:.2e}"
    print("  rel errors dq dk dv", " ".join(f"{e:.2e}" for e in errs), flush=True)


CASES = [
    # b, hq, hkv, lq, lk, dqk, dv, dtype, mask, window
    (1, 4, 4, 128, 128, 64, 64, "bf16", "none", 0),
    (1, 4, 2, 200, 200, 64, 64, "bf16", "causal", 0),
    (2, 4, 1, 77, 300, 128, 128, "f16", "causal", 0),
    (1, 2, 2, 150, 333, 96, 96, "bf16", "window", 37),
    (1, 8, 2, 130, 130, 128, 128, "bf16", "none", 0),
    (1, 2, 2, 100, 100, 32, 32, "f16", "causal", 0),
    (1, 4, 2, 1, 500, 128, 128, "bf16", "causal", 0),
    (1, 2, 1, 70, 70, 72, 72, "bf16", "none", 0),
    (1, 3, 1, 40, 90, 48, 40, "f16", "causal", 0),
    (1, 2, 2, 257, 257, 128, 128, "bf16", "window", 100),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) for x in c))
def test_bwd_cases(case):
    _say(case)
    check_bwd(case)


@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_bwd_negative_and_zero_scale(scale):
    _say("bwd scale", scale)
    check_bwd((1, 2, 1, 60, 90, 64, 64, "bf16", "causal", 0), scale=scale)


def test_bwd_is_deterministic():
    _say("bwd determinism")
    a, _ = run_bwd(1, 4, 2, 150, 150, 64, 64, torch.bfloat16, "causal", 0, 5)
    b, _ = run_bwd(1, 4, 2, 150, 150, 64, 64, torch.bfloat16, "causal", 0, 5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# dK/dV key tiles cut into row parts (float32 partials summed by a last
# kernel): forced counts, including more parts than a tile has row blocks
# (empty parts write zeros), and the planner's own choice at a grouped-query
# causal shape that gets parts.
PARTS = [
    (1, 8, 2, 300, 300, 64, 64, "bf16", "causal", 0),
    (1, 4, 1, 200, 333, 128, 128, "f16", "none", 0),
    (1, 4, 2, 260, 260, 96, 96, "bf16", "window", 70),
    (2, 6, 2, 130, 200, 32, 48, "f16", "causal", 0),
]


@pytest.mark.parametrize("parts", [1, 2, 3, 5, 16])
@pytest.mark.parametrize("case", PARTS, ids=lambda c: "-".join(str(x) for x in c))
def test_bwd_row_parts(case, parts):
    _say("bwd row parts", parts, case)
    check_bwd(case, kv_parts=parts)


def test_bwd_row_parts_auto_and_deterministic():
    """B=1, Hq=16, Hkv=4, L=2048, D=64, causal: the planner cuts each dK/dV
    key tile into row parts (64 tiles for 256 CUs); two runs agree bitwise."""
    _say("bwd row parts auto")
    d = sdpa.make_desc((1, 16, 2048, 64), (1, 4, 2048, 64), (1, 4, 2048, 64), sdpa.SDPA_BF16, mask="causal")
    d1 = sdpa.make_desc((1, 16, 2048, 64), (1, 4, 2048, 64), (1, 4, 2048, 64), sdpa.SDPA_BF16, mask="causal",
                        num_splits=1)
    assert sdpa.sdpa_backward_workspace_bytes(d) > sdpa.sdpa_backward_workspace_bytes(d1)
    case = (1, 16, 4, 2048, 2048, 64, 64, "bf16", "causal", 0)
    check_bwd(case)
    a, _ = run_bwd(1, 16, 4, 2048, 2048, 64, 64, torch.bfloat16, "causal", 0, 5)
    b, _ = run_bwd(1, 16, 4, 2048, 2048, 64, 64, torch.bfloat16, "causal", 0, 5)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bwd_causal_l1024_d128():
    """Training-size layer: B=1, Hq=8, Hkv=2, L=1024, D=128, causal."""
    _say("bwd causal L=1024 D=128")
    check_bwd((1, 8, 2, 1024, 1024, 128, 128, "bf16", "causal", 0))


# ---- per-batch lengths ----
# Positions past the lengths hold NaN in q, k, v and dout (and the forward
# leaves o / lse there unwritten, NaN): the backward must never read them,
# and every gradient position past the lengths must come back exactly 0.

VARLEN = [
    # b, hq, hkv, lq, lk, dqk, dv, dtype, mask, window, q_lens, kv_lens
    (3, 4, 2, 70, 300, 64, 64, "bf16", "causal", 0, [70, 5, 33], [300, 40, 0]),
    (2, 8, 2, 1, 700, 128, 128, "bf16", "none", 0, None, [700, 129]),
    (2, 4, 4, 150, 150, 96, 96, "f16", "causal", 0, [150, 77], [150, 100]),
    (2, 2, 1, 90, 260, 128, 128, "bf16", "window", 50, [90, 60], [260, 61]),
    (2, 4, 2, 40, 50, 32, 32, "f16", "causal", 0, [40, 30], [20, 50]),  # entry 0: more queries than keys
]


def _poison(x, lens, dim_len):
    """NaN at positions i >= lens[b] along dim 2 of a [B, H, L, D] tensor."""
    if lens is None:
        return x
    x = x.clone()
    for bi, n in enumerate(lens):
        x[bi, :, n:] = float("nan")
    return x


@pytest.mark.parametrize("case", VARLEN, ids=lambda c: "-".join(str(x) for x in c[:10]))
def test_bwd_varlen(case):
    from oracle import sdpa_bwd_ref_varlen

    b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, ql, kl = case
    _say("bwd varlen", case)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    seed = zlib.crc32(repr(case).encode()) % 10000
    q, k, v = make_qkv(b, hq, hkv, lq, lk, dqk, dv, dt, seed)
    do = randn((b, hq, lq, dv), seed + 3, dt)
    scale = default_scale(dqk)
    ref = sdpa_bwd_ref_varlen(q, k, v, do, scale, mask, w, ql, kl)
    dev = torch.device("cuda", 0)
    qd, dod = _poison(q, ql, lq).to(dev), _poison(do, ql, lq).to(dev)
    kd, vd = _poison(k, kl, lk).to(dev), _poison(v, kl, lk).to(dev)
    qt = None if ql is None else torch.tensor(ql, dtype=torch.int32, device=dev)
    kt = None if kl is None else torch.tensor(kl, dtype=torch.int32, device=dev)
    o = torch.full((b, hq, lq, dv), float("nan"), dtype=dt, device=dev)
    lse = torch.full((b, hq, lq), float("nan"), dtype=torch.float32, device=dev)
    sdpa.forward(qd, kd, vd, scale=scale, mask=mask, window_size=w, q_lens=qt, kv_lens=kt, return_lse=True,
                 out=o, lse_out=lse)
    grads = [torch.full_like(x, float("nan")) for x in (qd, kd, vd)]
    gq, gk, gv = sdpa.backward(qd, kd, vd, o, dod, lse, scale=scale, mask=mask, window_size=w, q_lens=qt,
                               kv_lens=kt, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    errs = []
    for name, g, r, lens in zip(("dq", "dk", "dv"), (gq, gk, gv), ref, (ql, kl, kl)):
        g = g.cpu().double().numpy()
        assert not np.isnan(g).any(), f"{name}: NaN (unwritten, or a padded position was read)"
        if lens is not None:
            for bi, n in enumerate(lens):
                assert (g[bi, :, n:] == 0).all(), f"{name}: non-zero gradient past the lengths of entry {bi}"
        scale_ref = max(float(np.abs(r).max()), 1e-30)
        e = float(np.abs(g - r).max()) / scale_ref
        errs.append(e)
        assert e <= TOL_REL[dt], f"{name}: max|g - ref| / max|ref| = {e:.3e} > {TOL_REL[dt]:.2e}"
    print("  rel errors dq dk dv", " ".join(f"{e:.2e}" for e in errs), flush=True)


# ---- explicit mask arrays ----

MASKED = [
    # b, hq, hkv, lq, lk, d, dtype, mode, window, mask shape, kind, q_lens, kv_lens
    (2, 4, 2, 96, 200, 64, "bf16", "causal", 0, (2, 1, 96, 200), "bool", None, None),
    (1, 4, 4, 130, 130, 128, "f16", "none", 0, (1, 4, 130, 130), "add", None, None),
    (2, 2, 1, 70, 260, 96, "bf16", "window", 60, (1, 1, 70, 260), "add", None, None),
    (2, 8, 2, 1, 513, 128, "bf16", "none", 0, (2, 1, 1, 513), "bool", None, None),
    (3, 4, 2, 40, 150, 64, "f16", "causal", 0, (3, 1, 40, 150), "bool", [40, 17, 40], [150, 90, 33]),
]


@pytest.mark.parametrize("case", MASKED, ids=lambda c: "-".join(str(x) for x in c[:11]))
def test_bwd_mask_array(case):
    from oracle import sdpa_bwd_ref_varlen
    from scaled_dot_product_fwd_amd.synth import additive_mask, bool_mask

    b, hq, hkv, lq, lk, d, dt, mode, w, mshape, kind, ql, kl = case
    _say("bwd mask array", case)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    seed = zlib.crc32(repr(case).encode()) % 10000
    q, k, v = make_qkv(b, hq, hkv, lq, lk, d, d, dt, seed)
    do = randn((b, hq, lq, d), seed + 3, dt)
    arr = bool_mask(mshape, seed + 5, keep=0.7) if kind == "bool" else additive_mask(mshape, seed + 5, dt)
    scale = default_scale(d)
    ref = sdpa_bwd_ref_varlen(q, k, v, do, scale, mode, w, ql, kl, mask_arr=arr)
    dev = torch.device("cuda", 0)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    md = sdpa.pad_mask(arr.to(dev))
    qt = None if ql is None else torch.tensor(ql, dtype=torch.int32, device=dev)
    kt = None if kl is None else torch.tensor(kl, dtype=torch.int32, device=dev)
    o, lse = sdpa.forward(qd, kd, vd, scale=scale, mask=mode, window_size=w, attn_mask=md, q_lens=qt,
                          kv_lens=kt, return_lse=True)
    grads = [torch.full_like(x, float("nan")) for x in (qd, kd, vd)]
    gq, gk, gv = sdpa.backward(qd, kd, vd, o, dod, lse, scale=scale, mask=mode, window_size=w, attn_mask=md,
                               q_lens=qt, kv_lens=kt, dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), (gq, gk, gv), ref):
        g = g.cpu().double().numpy()
        assert not np.isnan(g).any(), f"{name}: NaN"
        scale_ref = max(float(np.abs(r).max()), 1e-30)
        e = float(np.abs(g - r).max()) / scale_ref
        errs.append(e)
        assert e <= TOL_REL[dt], f"{name}: max|g - ref| / max|ref| = {e:.3e} > {TOL_REL[dt]:.2e}"
    print("  rel errors dq dk dv", " ".join(f"{e:.2e}" for e in errs), flush=True)
