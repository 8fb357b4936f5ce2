"""GPU parity of the fused forward with explicit mask arrays (boolean: True
keeps a key; additive: added to the scaled scores), against the float64
oracle on the same seeded inputs.

Cases cover every kernel family (prefill, short, decode), the three element
types, ragged key lengths (rows padded to 16 bytes by pad_mask), broadcast
mask shapes ([Lq, Lk], [B, 1, 1, Lk], [1, Hq, Lq, Lk], full) and combination
with the causal and window modes.  Rows that keep no key must give o = 0 and
lse = -inf on every plan (unsplit, split + combine, cross-wave merge).
"""

import zlib

import numpy as np
import pytest
import torch

import scaled_dot_product_fwd_amd as sdpa
from gpu_cases import TOL_LSE, TOL_O, check_full, check_sampled, lse_err, run_gpu, to_dtype
from oracle import sdpa_ref, visible_mask
from scaled_dot_product_fwd_amd.synth import (additive_mask, bool_mask, default_scale, make_qkv,
                                              padding_mask)

pytestmark = pytest.mark.gpu


def _say(*a):
    print("CASE", *a, flush=True)


def _mask(kind, shape, seed, dtype):
    if kind == "bool":
        return bool_mask(shape, seed, keep=0.7)
    return additive_mask(shape, seed, to_dtype(dtype))


MASK_CASES = [
    # b, hq, hkv, lq, lk, dqk, dv, dtype, mode, window, kind, mask shape
    (1, 4, 2, 200, 333, 64, 64, "bf16", "none", 0, "bool", (200, 333)),
    (1, 4, 2, 200, 333, 64, 64, "bf16", "none", 0, "add", (200, 333)),
    (2, 4, 1, 130, 257, 128, 128, "f16", "causal", 0, "add", (2, 4, 130, 257)),
    (1, 4, 4, 150, 150, 128, 128, "bf16", "causal", 0, "bool", (1, 4, 150, 150)),
    (2, 2, 2, 140, 300, 256, 256, "bf16", "window", 70, "add", (2, 1, 1, 300)),
    (1, 2, 2, 140, 300, 256, 256, "bf16", "none", 0, "bool", (140, 300)),
    (1, 8, 2, 100, 100, 72, 72, "bf16", "none", 0, "add", (100, 100)),
    (1, 4, 2, 200, 333, 80, 80, "f16", "causal", 0, "bool", (1, 4, 200, 333)),
    (1, 16, 4, 1, 1200, 72, 72, "bf16", "none", 0, "bool", (1, 16, 1, 1200)),
    (1, 32, 8, 48, 700, 72, 72, "bf16", "none", 0, "add", (48, 700)),
    (1, 2, 1, 129, 129, 160, 160, "f16", "none", 0, "bool", (1, 2, 129, 129)),
    (1, 2, 2, 96, 96, 16, 48, "f16", "causal", 0, "bool", (96, 96)),
    (1, 2, 2, 130, 200, 192, 128, "bf16", "causal", 0, "add", (130, 200)),
    (1, 16, 1, 3, 777, 192, 128, "bf16", "causal", 0, "bool", (1, 16, 3, 777)),
    (1, 4, 1, 12, 1500, 128, 128, "f16", "causal", 0, "add", (12, 1500)),
    (1, 4, 1, 12, 1500, 224, 224, "bf16", "none", 0, "bool", (1, 4, 12, 1500)),
    (1, 32, 8, 1, 1000, 128, 128, "bf16", "none", 0, "bool", (1, 32, 1, 1000)),
    (1, 32, 8, 1, 2000, 128, 128, "f16", "none", 0, "add", (1, 1, 1, 2000)),
    (1, 32, 8, 1, 2000, 160, 160, "bf16", "none", 0, "add", (1, 32, 1, 2000)),
    (1, 8, 2, 1, 4096, 32, 64, "f32", "none", 0, "add", (1, 8, 1, 4096)),
    (1, 4, 2, 64, 190, 64, 64, "f32", "causal", 0, "bool", (64, 190)),
    (2, 4, 2, 70, 190, 128, 128, "f32", "window", 50, "add", (2, 4, 70, 190)),
    (1, 4, 4, 33, 45, 96, 96, "f32", "none", 0, "bool", (33, 45)),
]


@pytest.mark.parametrize("case", MASK_CASES, ids=lambda c: "-".join(str(x) for x in c[:11]))
def test_mask_array_cases(case):
    b, hq, hkv, lq, lk, dqk, dv, dt, mode, w, kind, shape = case
    _say(case)
    seed = zlib.crc32(repr(case).encode()) % 10000
    check_full(b, hq, hkv, lq, lk, dqk, dv, dt, mode, w, seed=seed,
               attn_mask=_mask(kind, shape, seed + 5, dt))


@pytest.mark.parametrize("splits", [1, 3, 16])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_mask_array_forced_splits(splits, kind):
    _say("mask splits", splits, kind)
    check_full(1, 16, 4, 1, 3000, 128, 128, "bf16", "none", 0, seed=31 + splits,
               attn_mask=_mask(kind, (1, 16, 1, 3000), 77, "bf16"), num_splits=splits)


@pytest.mark.parametrize("row_tile", [32, 64, 128])
def test_mask_array_forced_row_tiles(row_tile):
    _say("mask row tile", row_tile)
    check_full(1, 4, 2, 90, 260, 128, 128, "bf16", "causal", 0, seed=41,
               attn_mask=_mask("bool", (1, 4, 90, 260), 78, "bf16"), row_tile=row_tile)


@pytest.mark.parametrize("plan", [dict(), dict(num_splits=4), dict(row_tile=128)],
                         ids=["auto", "splits4", "prefill-tile"])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_rows_without_keys_give_zero_and_minus_inf(plan, kind):
    """Whole rows removed by the array: o = 0 and lse = -inf, and the other
    rows unaffected, on the decode plan (cross-wave merge), a split plan
    (combine) and a prefill tile."""
    _say("empty rows", plan, kind)
    b, hq, hkv, lq, lk = 1, 8, 2, 6, 700
    keep = bool_mask((b, hq, lq, lk), 5, keep=0.8)
    keep[0, 0, 0] = False
    keep[0, 3, 2] = False
    keep[0, 7] = False  # every row of head 7
    arr = keep if kind == "bool" else torch.where(keep, torch.tensor(0.25), torch.tensor(float("-inf"))).to(
        torch.bfloat16)
    q, k, v = make_qkv(b, hq, hkv, lq, lk, 64, 64, torch.bfloat16, 9)
    scale = default_scale(64)
    o, lse = run_gpu(q, k, v, scale, "none", 0, attn_mask=arr, **plan)
    ro, rl = sdpa_ref(q, k, v, scale, "none", 0, mask_arr=arr)
    empty = ~keep.numpy().any(axis=-1)
    assert empty[0, 0, 0] and empty[0, 7].all()
    assert (o[empty] == 0.0).all()
    assert np.isneginf(lse[empty]).all()
    assert float(np.abs(o - ro).max()) <= TOL_O[torch.bfloat16]
    assert lse_err(lse, rl) <= TOL_LSE[torch.bfloat16]


def test_window_array_matches_window_mode():
    """A window spelled as an explicit [Lq, Lk] boolean array (no mode) gives
    the window mode's result."""
    _say("window as array")
    b, hq, hkv, lq, lk, d, w = 1, 4, 2, 300, 300, 128, 64
    q, k, v = make_qkv(b, hq, hkv, lq, lk, d, d, torch.bfloat16, 12)
    scale = default_scale(d)
    arr = torch.from_numpy(visible_mask(lq, lk, "window", w))
    o1, l1 = run_gpu(q, k, v, scale, "window", w)
    o2, l2 = run_gpu(q, k, v, scale, "none", 0, attn_mask=arr)
    ro, rl = sdpa_ref(q, k, v, scale, "window", w)
    assert float(np.abs(o2 - ro).max()) <= TOL_O[torch.bfloat16]
    assert float(np.abs(l2 - rl).max()) <= TOL_LSE[torch.bfloat16]
    assert float(np.abs(o1 - o2).max()) <= TOL_O[torch.bfloat16]


def test_mask_array_strided_view_and_uint8():
    """A uint8 mask read through a strided view of a larger padded buffer."""
    _say("uint8 strided mask")
    b, hq, hkv, lq, lk = 2, 4, 2, 50, 120
    keep = bool_mask((b, hq, lq, lk), 13, keep=0.6)
    keep[..., 0] = True
    dev = torch.device("cuda", 0)
    big = torch.zeros((b, hq, lq + 3, 160), dtype=torch.uint8, device=dev)
    big[:, :, 3:, :lk] = keep.to(torch.uint8).to(dev)
    view = big[:, :, 3:, :lk]
    q, k, v = make_qkv(b, hq, hkv, lq, lk, 64, 64, torch.float16, 14)
    scale = default_scale(64)
    o = sdpa.forward(q.to(dev), k.to(dev), v.to(dev), scale=scale, attn_mask=view)
    ro, _ = sdpa_ref(q, k, v, scale, "none", 0, mask_arr=keep)
    assert float(np.abs(o.cpu().double().numpy() - ro).max()) <= TOL_O[torch.float16]


def test_padding_mask_decode_sampled():
    """Decode with a key-padding mask [B, 1, 1, Lk] per batch entry, at a
    serving size; the oracle recomputes sampled rows."""
    _say("padding mask decode B=4 Hq=32 Hkv=8 Lk=8192")
    check_sampled(4, 32, 8, 1, 8192, 128, 128, "bf16", "none", 0, seed=91, nrows=24,
                  attn_mask=padding_mask(4, 8192, 3, min_len=1000))


def test_window_array_prefill_sampled():
    """Prefill L=4096 with a 1024-key window spelled as a [L, L] boolean array."""
    _say("window array prefill L=4096 W=1024")
    L = 4096
    check_sampled(1, 8, 8, L, L, 128, 128, "bf16", "none", 0, seed=92, nrows=24,
                  attn_mask=torch.from_numpy(visible_mask(L, L, "window", 1024)))


def test_additive_bias_causal_prefill_sampled():
    """Causal prefill L=2048 with a per-head additive bias [1, Hq, L, L]."""
    _say("additive bias causal prefill L=2048")
    L = 2048
    check_sampled(1, 8, 2, L, L, 128, 128, "bf16", "causal", 0, seed=93, nrows=24,
                  attn_mask=additive_mask((1, 8, L, L), 94, torch.bfloat16, sigma=1.0, minus_inf=0.0))


@pytest.mark.parametrize("dt,d", [("bf16", 64), ("f16", 128), ("f32", 64), ("bf16", 256)])
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_blocks_removed_by_the_array_are_skipped_exactly(dt, d, kind):
    """A band mask leaves whole key blocks without a kept key (the kernel
    skips their products): the result still matches the oracle, for the
    pipelined small-dim loop and the plain loop, both array kinds."""
    _say("dead blocks", dt, d, kind)
    L, w = 400, 48
    band = torch.from_numpy(visible_mask(L, L, "window", w))
    arr = band if kind == "bool" else torch.where(band, torch.tensor(0.5), torch.tensor(float("-inf"))).to(
        to_dtype(dt))
    check_full(1, 2, 1, L, L, d, d, dt, "none", 0, seed=d, attn_mask=arr)


@pytest.mark.parametrize("kind", ["bool", "add"])
def test_mask_array_wide_family(kind):
    _say("wide + mask array", kind)
    check_full(1, 32, 8, 48, 700, 128, 128, "bf16", "causal", 0, seed=61,
               attn_mask=_mask(kind, (1, 32, 48, 700), 62, "bf16"))
