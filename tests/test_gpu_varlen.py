"""GPU parity with per-batch lengths (q_lens / kv_lens device arrays) against
the float64 oracle's sdpa_ref_varlen on the same seeded inputs.

Entry b uses its first q_lens[b] queries and kv_lens[b] keys, query i at key
position i + kv_lens[b] - q_lens[b].  Rows past q_lens[b] must stay untouched
(the outputs are poisoned with NaN before the call); rows with no visible key
give 0 / -inf.
"""

import zlib

import numpy as np
import pytest
import torch

import scaled_dot_product_fwd_amd as sdpa
from gpu_cases import TOL_LSE, TOL_O, lse_err, pick_rows, to_dtype
from oracle import sdpa_ref_rows, sdpa_ref_varlen
from scaled_dot_product_fwd_amd.synth import bool_mask, default_scale, make_qkv

pytestmark = pytest.mark.gpu


def _say(*a):
    print("CASE", *a, flush=True)


def _run(b, hq, hkv, lq, lk, dqk, dv, dt, mode, w, ql, kl, seed, attn_mask=None, **plan):
    dt = to_dtype(dt)
    q, k, v = make_qkv(b, hq, hkv, lq, lk, dqk, dv, dt, seed)
    scale = default_scale(dqk)
    dev = torch.device("cuda", 0)
    out = torch.full((b, hq, lq, dv), float("nan"), dtype=dt, device=dev)
    lse = torch.full((b, hq, lq), float("nan"), dtype=torch.float32, device=dev)
    qt = None if ql is None else torch.tensor(ql, dtype=torch.int32, device=dev)
    kt = None if kl is None else torch.tensor(kl, dtype=torch.int32, device=dev)
    if attn_mask is not None:
        plan["attn_mask"] = sdpa.pad_mask(attn_mask.to(dev))
    sdpa.forward(q.to(dev), k.to(dev), v.to(dev), scale=scale, mask=mode, window_size=w, q_lens=qt,
                 kv_lens=kt, return_lse=True, out=out, lse_out=lse, **plan)
    torch.cuda.synchronize()
    return (q, k, v, scale, out.cpu().double().numpy(), lse.cpu().double().numpy())


def _check(case, attn_mask=None, **plan):
    b, hq, hkv, lq, lk, dqk, dv, dt, mode, w, ql, kl = case
    seed = zlib.crc32(repr(case).encode()) % 10000
    q, k, v, scale, o, lse = _run(b, hq, hkv, lq, lk, dqk, dv, dt, mode, w, ql, kl, seed, attn_mask, **plan)
    ro, rl = sdpa_ref_varlen(q, k, v, scale, mode, w, ql, kl, mask_arr=attn_mask)
    valid = ~np.isnan(rl)  # rows below q_lens[b]
    assert (np.isnan(o[~valid]).all() and np.isnan(lse[~valid]).all()), "rows past q_lens were written"
    assert not np.isnan(o[valid]).any() and not np.isnan(lse[valid]).any(), "unwritten valid rows"
    dtt = to_dtype(dt)
    eo = float(np.abs(o[valid] - ro[valid]).max()) if valid.any() else 0.0
    el = lse_err(lse[valid], rl[valid])
    assert eo <= TOL_O[dtt], f"max|o - ref| = {eo:.3e}"
    assert el <= TOL_LSE[dtt], f"max|lse - ref| = {el:.3e}"


CASES = [
    # b, hq, hkv, lq, lk, dqk, dv, dtype, mode, window, q_lens, kv_lens
    (4, 32, 8, 1, 2000, 128, 128, "bf16", "none", 0, None, [2000, 1, 0, 777]),
    (4, 16, 4, 1, 3000, 192, 128, "bf16", "causal", 0, None, [3000, 65, 1000, 2999]),
    (3, 8, 2, 8, 1500, 128, 128, "f16", "causal", 0, [8, 3, 0], [1500, 600, 100]),
    (2, 4, 2, 200, 700, 64, 64, "bf16", "causal", 0, [200, 130], [700, 260]),
    (2, 2, 2, 140, 500, 256, 256, "bf16", "causal", 0, [140, 77], [500, 300]),
    (2, 4, 1, 150, 400, 96, 96, "bf16", "window", 37, [150, 100], [400, 90]),
    (2, 4, 2, 70, 190, 128, 128, "f32", "causal", 0, [70, 33], [190, 40]),
    (3, 4, 4, 64, 300, 64, 64, "f16", "none", 0, [64, 1, 50], [1, 300, 128]),
    (2, 8, 8, 5, 400, 192, 192, "f16", "causal", 0, [5, 5], [5, 2]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) for x in c[:10]))
def test_varlen_cases(case):
    _say(case)
    _check(case)


@pytest.mark.parametrize("splits", [1, 8, 32])
def test_varlen_forced_splits(splits):
    case = (3, 16, 4, 2, 4000, 128, 128, "bf16", "causal", 0, [2, 1, 2], [4000, 100, 0])
    _say("varlen splits", splits)
    _check(case, num_splits=splits)


def test_varlen_with_mask_array():
    case = (2, 4, 2, 90, 300, 128, 128, "bf16", "causal", 0, [90, 40], [300, 120])
    _say("varlen + bool mask")
    _check(case, attn_mask=bool_mask((2, 1, 90, 300), 4, keep=0.7))


def test_varlen_only_q_lens():
    case = (2, 4, 2, 100, 100, 64, 64, "bf16", "causal", 0, [100, 31], None)
    _say("q_lens only")
    _check(case)


def test_varlen_decode_sampled_full_size():
    """Serving-size varlen decode: B=8, Hq=32, Hkv=8, cache 8192, lengths
    spread over the cache; the oracle recomputes sampled rows."""
    b, hq, hkv, lk, d = 8, 32, 8, 8192, 128
    kl = [8192, 1, 4097, 6000, 2048, 8191, 300, 5000]
    _say("varlen decode B=8 cache 8192")
    q, k, v, scale, o, lse = _run(b, hq, hkv, 1, lk, d, d, "bf16", "none", 0, None, kl, 77)
    picks = pick_rows(b, hq, 1, 48, 5)
    ro, rl = sdpa_ref_rows(q, k, v, scale, "none", 0, picks, kv_lens=kl)
    go = np.stack([o[p] for p in picks])
    gl = np.array([lse[p] for p in picks])
    assert float(np.abs(go - ro).max()) <= TOL_O[torch.bfloat16]
    assert lse_err(gl, rl) <= TOL_LSE[torch.bfloat16]


def test_varlen_head_dim_512():
    case = (2, 8, 2, 4, 900, 512, 512, "bf16", "causal", 0, [4, 2], [900, 130])
    _say("varlen d512")
    _check(case)


def test_varlen_wide_family():
    case = (2, 32, 8, 48, 1200, 128, 128, "bf16", "causal", 0, [48, 20], [1200, 300])
    _say("varlen wide")
    _check(case)


@pytest.mark.parametrize("splits", [0, 4, 16, 1024])
def test_varlen_balanced_deal(splits):
    """Split plans with kv_lens deal each KV head's workgroups to the entries
    by their key blocks: skewed lengths, an empty entry, entries shorter than
    one block and more splits than blocks must all merge back exactly."""
    case = (6, 8, 2, 1, 5000, 128, 128, "bf16", "none", 0, None, [5000, 3, 0, 4999, 64, 2500])
    _say("varlen balanced deal", splits)
    _check(case, num_splits=splits)


def test_varlen_balanced_deal_causal_rows():
    case = (4, 8, 2, 6, 3000, 64, 64, "f16", "causal", 0, [6, 2, 6, 1], [3000, 40, 6, 1777])
    _say("varlen balanced deal causal")
    _check(case, num_splits=24)


def test_varlen_balanced_deal_many_entries():
    """Forty entries, most of them with a share of one or two workgroups:
    lengths from 0 to the full cache."""
    rng = np.random.default_rng(2024)
    kl = [int(x) for x in rng.integers(0, 2049, size=40)]
    kl[3], kl[17], kl[39] = 0, 2048, 1
    case = (40, 8, 2, 1, 2048, 64, 64, "f16", "none", 0, None, kl)
    _say("varlen balanced deal, 40 entries")
    _check(case)
