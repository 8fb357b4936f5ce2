"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: a pure-Python loop
formulation on tiny inputs, closed forms, invariants, a library special case
(torch's CPU float64 attention with an explicit boolean mask) and the K-block
skip ratios printed in mlx PR #3552 "feat(fast): add sliding-window SDPA kernel
path" (Performance table), stored under ``tests/golden/``.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch

from oracle import (sdpa_loop, sdpa_probs, sdpa_ref, sdpa_ref_rows, visible_mask,
                    visible_pairs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(b, hq, hkv, lq, lk, dqk, dv, seed):
    return (_rand((b, hq, lq, dqk), seed), _rand((b, hkv, lk, dqk), seed + 1),
            _rand((b, hkv, lk, dv), seed + 2))


TINY = [
    # b, hq, hkv, lq, lk, dqk, dv, mask, window
    (1, 2, 2, 3, 5, 4, 4, "none", 0),
    (2, 4, 2, 5, 5, 3, 6, "none", 0),
    (1, 4, 1, 1, 7, 5, 2, "none", 0),
    (1, 2, 1, 4, 4, 4, 4, "causal", 0),
    (2, 4, 2, 3, 7, 6, 3, "causal", 0),
    (1, 3, 3, 1, 6, 2, 5, "causal", 0),
    (1, 2, 1, 6, 6, 4, 4, "window", 1),
    (1, 4, 2, 5, 9, 3, 4, "window", 3),
    (2, 2, 2, 4, 4, 4, 2, "window", 2),
    (1, 2, 1, 3, 8, 5, 5, "window", 20),
]


@pytest.mark.parametrize("case", TINY)
def test_ref_matches_loop_brute_force(case):
    b, hq, hkv, lq, lk, dqk, dv, mask, w = case
    q, k, v = _case(b, hq, hkv, lq, lk, dqk, dv, seed=sum(case[:7]))
    o, lse = sdpa_ref(q, k, v, 0.7, mask, w)
    o2, lse2 = sdpa_loop(q, k, v, 0.7, mask, w)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", TINY)
def test_ref_rows_matches_ref(case):
    b, hq, hkv, lq, lk, dqk, dv, mask, w = case
    q, k, v = _case(b, hq, hkv, lq, lk, dqk, dv, seed=3 + sum(case[:7]))
    o, lse = sdpa_ref(q, k, v, 1.3, mask, w)
    picks = list(itertools.product(range(b), range(hq), range(lq)))
    orow, lrow = sdpa_ref_rows(q, k, v, 1.3, mask, w, picks)
    for n, (bi, h, i) in enumerate(picks):
        np.testing.assert_allclose(orow[n], o[bi, h, i], rtol=0, atol=1e-12)
        assert abs(lrow[n] - lse[bi, h, i]) < 1e-12


@pytest.mark.parametrize("case", TINY)
def test_torch_cpu_sdpa_special_case(case):
    """Library special case: torch's float64 CPU attention, explicit bool mask, KV heads repeated."""
    b, hq, hkv, lq, lk, dqk, dv, mask, w = case
    q, k, v = _case(b, hq, hkv, lq, lk, dqk, dv, seed=11 + sum(case[:7]))
    o, _ = sdpa_ref(q, k, v, 0.45, mask, w)
    g = hq // hkv
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1)
    m = torch.from_numpy(visible_mask(lq, lk, mask, w))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=0.45)
    np.testing.assert_allclose(o, ot.numpy(), rtol=0, atol=1e-12)


def _expected_visible_set(i, lq, lk, mask, w):
    """Textbook statement of the visible key set of query row i (bottom-right aligned)."""
    last = lk - lq + i  # the key position the query occupies
    if mask == "none":
        return set(range(lk))
    if mask == "causal":
        return set(range(0, last + 1))
    return set(range(max(0, last - w + 1), last + 1))


@pytest.mark.parametrize("lq,lk,mask,w", [
    (1, 9, "causal", 0), (4, 9, "causal", 0), (9, 9, "causal", 0), (5, 9, "none", 0),
    (9, 9, "window", 1), (9, 9, "window", 4), (3, 11, "window", 5), (6, 6, "window", 6),
    (2, 7, "window", 100),
])
def test_zero_query_identity_values_reveal_visible_set(lq, lk, mask, w):
    """Q = 0 makes every visible key equally likely: with V = I the output row is
    the indicator of the visible set over its size, and lse = ln(size)."""
    q = np.zeros((1, 1, lq, 3))
    k = _rand((1, 1, lk, 3), 5)
    v = np.eye(lk)[None, None]
    o, lse = sdpa_ref(q, k, v, 1.0, mask, w)
    for i in range(lq):
        vis = _expected_visible_set(i, lq, lk, mask, w)
        exp = np.array([1.0 / len(vis) if j in vis else 0.0 for j in range(lk)])
        np.testing.assert_allclose(o[0, 0, i], exp, rtol=0, atol=1e-15)
        assert abs(lse[0, 0, i] - math.log(len(vis))) < 1e-14


def test_scale_zero_gives_mean_of_values():
    q, k, v = _case(1, 2, 1, 4, 6, 5, 3, seed=21)
    o, lse = sdpa_ref(q, k, v, 0.0, "causal", 0)
    for i in range(4):
        n = i + 2 + 1
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, :n].mean(axis=0), atol=1e-14)
        assert abs(lse[0, 1, i] - math.log(n)) < 1e-14


def test_single_key_closed_form():
    q, k, v = _case(1, 3, 1, 1, 1, 4, 5, seed=31)
    o, lse = sdpa_ref(q, k, v, 0.37, "none", 0)
    for h in range(3):
        np.testing.assert_allclose(o[0, h, 0], v[0, 0, 0], atol=1e-15)
        assert abs(lse[0, h, 0] - 0.37 * float(q[0, h, 0] @ k[0, 0, 0])) < 1e-13


def test_two_keys_sigmoid_closed_form():
    q, k, v = _case(1, 1, 1, 3, 2, 4, 3, seed=41)
    o, lse = sdpa_ref(q, k, v, 0.8, "none", 0)
    for i in range(3):
        s0 = 0.8 * float(q[0, 0, i] @ k[0, 0, 0])
        s1 = 0.8 * float(q[0, 0, i] @ k[0, 0, 1])
        sig = 1.0 / (1.0 + math.exp(-(s0 - s1)))
        np.testing.assert_allclose(o[0, 0, i], sig * v[0, 0, 0] + (1 - sig) * v[0, 0, 1], atol=1e-14)
        assert abs(lse[0, 0, i] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-13


def test_window_one_selects_own_position():
    q, k, v = _case(1, 2, 2, 4, 7, 3, 4, seed=51)
    o, lse = sdpa_ref(q, k, v, 2.0, "window", 1)
    for h in range(2):
        for i in range(4):
            p = i + 3
            np.testing.assert_allclose(o[0, h, i], v[0, h, p], atol=1e-15)
            assert abs(lse[0, h, i] - 2.0 * float(q[0, h, i] @ k[0, h, p])) < 1e-13


def test_large_scale_limit_picks_argmax():
    q, k, v = _case(1, 1, 1, 4, 16, 8, 4, seed=61)
    o, _ = sdpa_ref(q, k, v, 1e4, "none", 0)
    s = q[0, 0] @ k[0, 0].T
    for i in range(4):
        np.testing.assert_allclose(o[0, 0, i], v[0, 0, int(np.argmax(s[i]))], atol=1e-9)


@pytest.mark.parametrize("mask,w", [("none", 0), ("causal", 0), ("window", 3)])
def test_probabilities_sum_to_one_and_reproduce_output(mask, w):
    q, k, v = _case(2, 4, 2, 5, 8, 6, 3, seed=71)
    p = sdpa_probs(q, k, 0.5, mask, w)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-14)
    assert (p[..., ~visible_mask(5, 8, mask, w)] == 0).all()
    o, _ = sdpa_ref(q, k, v, 0.5, mask, w)
    g = 2
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(p[b, h] @ v[b, h // g], o[b, h], atol=1e-13)


def test_output_linear_in_values():
    q, k, v1 = _case(1, 2, 1, 4, 6, 4, 3, seed=81)
    v2 = _rand(v1.shape, 82)
    a, c = 0.3, -1.7
    o1, _ = sdpa_ref(q, k, v1, 0.9, "causal", 0)
    o2, _ = sdpa_ref(q, k, v2, 0.9, "causal", 0)
    o3, _ = sdpa_ref(q, k, a * v1 + c * v2, 0.9, "causal", 0)
    np.testing.assert_allclose(o3, a * o1 + c * o2, atol=1e-13)


def test_unmasked_invariant_to_key_permutation():
    q, k, v = _case(1, 2, 2, 3, 9, 4, 4, seed=91)
    perm = np.random.default_rng(0).permutation(9)
    o, lse = sdpa_ref(q, k, v, 0.6, "none", 0)
    o2, lse2 = sdpa_ref(q, k[:, :, perm], v[:, :, perm], 0.6, "none", 0)
    np.testing.assert_allclose(o, o2, atol=1e-13)
    np.testing.assert_allclose(lse, lse2, atol=1e-13)


def test_causal_single_query_equals_no_mask():
    q, k, v = _case(1, 4, 2, 1, 10, 5, 3, seed=101)
    np.testing.assert_array_equal(sdpa_ref(q, k, v, 0.4, "causal")[0], sdpa_ref(q, k, v, 0.4, "none")[0])


@pytest.mark.parametrize("w", [9, 10, 1000])
def test_window_at_least_lk_equals_causal(w):
    q, k, v = _case(1, 2, 1, 6, 9, 4, 4, seed=111)
    a = sdpa_ref(q, k, v, 0.5, "causal")
    b = sdpa_ref(q, k, v, 0.5, "window", w)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_gqa_equals_repeated_kv_heads_bitwise():
    q, k, v = _case(2, 6, 2, 4, 7, 5, 3, seed=121)
    o, lse = sdpa_ref(q, k, v, 0.5, "causal")
    o2, lse2 = sdpa_ref(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.5, "causal")
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_gqa_uses_consecutive_heads():
    """Query heads 0..G-1 read KV head 0: zeroing KV head 1 leaves them unchanged."""
    q, k, v = _case(1, 4, 2, 3, 5, 4, 4, seed=131)
    o, _ = sdpa_ref(q, k, v, 0.5, "none")
    k2, v2 = k.copy(), v.copy()
    k2[:, 1] = 0
    v2[:, 1] = 0
    o2, _ = sdpa_ref(q, k2, v2, 0.5, "none")
    np.testing.assert_array_equal(o[:, :2], o2[:, :2])
    assert not np.allclose(o[:, 2:], o2[:, 2:])


def test_zero_padding_head_dims():
    q, k, v = _case(1, 2, 1, 4, 6, 5, 3, seed=141)
    o, lse = sdpa_ref(q, k, v, 0.5, "causal")
    pad = ((0, 0), (0, 0), (0, 0), (0, 3))
    o2, lse2 = sdpa_ref(np.pad(q, pad), np.pad(k, pad), np.pad(v, pad), 0.5, "causal")
    np.testing.assert_allclose(o2[..., :3], o, atol=1e-14)
    np.testing.assert_array_equal(o2[..., 3:], 0.0)
    np.testing.assert_allclose(lse2, lse, atol=1e-14)


@pytest.mark.parametrize("lq,lk,mask,w", [(7, 7, "none", 0), (7, 7, "causal", 0), (3, 10, "causal", 0),
                                         (10, 10, "window", 4), (4, 12, "window", 3), (5, 5, "window", 9)])
def test_visible_pair_counts_closed_form(lq, lk, mask, w):
    off = lk - lq
    if mask == "none":
        exp = lq * lk
    elif mask == "causal":
        exp = lq * (lq + 1) // 2 + lq * off
    else:
        exp = sum(min(w, i + off + 1) for i in range(lq))
    assert visible_pairs(lq, lk, mask, w) == exp


def _load_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_window_skip_ratio_matches_printed_table():
    """The K-block skip ratio printed for W=1024 at 2K/4K/8K is the fraction of the
    key range lying below the last query's window: (L - W) / L."""
    rows = _load_golden("window_skip_ratio.txt")
    assert len(rows) == 3
    for ctx, w, pct in rows:
        L, W = int(ctx), int(w)
        vis_last = visible_mask(4, L, "window", W)[-1]  # last query sits at position L-1
        below = int(np.argmax(vis_last))  # first visible key
        assert abs(100.0 * below / L - float(pct)) < 1e-9


@pytest.mark.parametrize("bad", [
    dict(lq=5, lk=4, mask="causal", w=0), dict(lq=5, lk=4, mask="window", w=2),
    dict(lq=2, lk=4, mask="window", w=0), dict(lq=2, lk=4, mask="bogus", w=0),
])
def test_invalid_masks_raise(bad):
    with pytest.raises(ValueError):
        visible_mask(bad["lq"], bad["lk"], bad["mask"], bad["w"])


def test_no_visible_keys_never_happens():
    for lq, lk in [(1, 1), (3, 3), (2, 9)]:
        for mask, w in [("causal", 0), ("window", 1), ("window", 2)]:
            assert visible_mask(lq, lk, mask, w).any(axis=1).all()


def test_oracle_reads_torch_low_precision_exactly():
    t = torch.tensor([1.0 + 2 ** -7, 3.140625, -0.0078125], dtype=torch.bfloat16)
    q = t.reshape(1, 1, 1, 3)
    o, lse = sdpa_ref(q, q, q, 1.0, "none")
    np.testing.assert_array_equal(o[0, 0, 0], np.array([1.0 + 2 ** -7, 3.140625, -0.0078125]))


# ---------------------------------------------------------------------------
# Explicit mask arrays (boolean: True keeps a key; float: added to the scaled
# score).  Pinned against the loop formulation, torch's CPU float64 attention
# with the same array (a library special case), closed forms and invariants.
# ---------------------------------------------------------------------------

MASKED = [
    # b, hq, hkv, lq, lk, dqk, dv, mode, window, mask shape (broadcast dims as 1)
    (1, 2, 1, 3, 5, 4, 4, "none", 0, (3, 5)),
    (2, 4, 2, 4, 6, 3, 5, "none", 0, (2, 4, 4, 6)),
    (2, 4, 2, 4, 6, 3, 5, "none", 0, (2, 1, 1, 6)),
    (1, 4, 1, 5, 7, 5, 3, "causal", 0, (1, 4, 5, 7)),
    (2, 2, 2, 3, 8, 4, 2, "window", 3, (3, 8)),
]


def _bool_mask(shape, seed, keep=0.6):
    return np.random.default_rng(seed).random(shape) < keep


def _add_mask(shape, seed):
    a = np.random.default_rng(seed).standard_normal(shape) * 2.0
    a[np.random.default_rng(seed + 1).random(shape) < 0.25] = -np.inf
    return a


def _torch_sdpa(q, k, v, scale, attn_mask):
    g = q.shape[1] // k.shape[1]
    tk = torch.from_numpy(k).repeat_interleave(g, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(g, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), tk, tv, attn_mask=torch.from_numpy(np.ascontiguousarray(attn_mask)),
        scale=scale).numpy()


@pytest.mark.parametrize("case", MASKED)
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_mask_array_matches_loop_brute_force(case, kind):
    b, hq, hkv, lq, lk, dqk, dv, mode, w, shape = case
    q, k, v = _case(b, hq, hkv, lq, lk, dqk, dv, seed=200 + lq + lk)
    arr = _bool_mask(shape, 7) if kind == "bool" else _add_mask(shape, 7)
    o, lse = sdpa_ref(q, k, v, 0.6, mode, w, mask_arr=arr)
    o2, lse2 = sdpa_loop(q, k, v, 0.6, mode, w, mask_arr=arr)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", MASKED)
@pytest.mark.parametrize("kind", ["bool", "add"])
def test_mask_array_matches_torch_cpu_sdpa(case, kind):
    """torch's float64 CPU attention takes the same array: boolean True keeps a
    key, a float array is added to the scaled scores.  The mode's own rule is
    written out here with index loops and folded into the array."""
    b, hq, hkv, lq, lk, dqk, dv, mode, w, shape = case
    q, k, v = _case(b, hq, hkv, lq, lk, dqk, dv, seed=300 + lq + lk)
    rule = np.ones((lq, lk), dtype=bool)
    for i in range(lq):
        for j in range(lk):
            p = i + lk - lq
            if mode != "none" and j > p:
                rule[i, j] = False
            if mode == "window" and j <= p - w:
                rule[i, j] = False
    if kind == "bool":
        arr = _bool_mask(shape, 9, keep=0.7)
        full = np.broadcast_to(arr, (b, hq, lq, lk)) & rule
        full = full | ~full.any(axis=-1, keepdims=True) & rule  # no empty row (torch gives NaN there)
        arr = full
        tmask = full
    else:
        arr = np.random.default_rng(9).standard_normal(shape) * 3.0
        tmask = np.where(rule, np.broadcast_to(arr, (b, hq, lq, lk)), -np.inf)
    o, lse = sdpa_ref(q, k, v, 0.45, mode, w, mask_arr=arr)
    np.testing.assert_allclose(o, _torch_sdpa(q, k, v, 0.45, tmask), rtol=0, atol=1e-12)


def test_additive_row_constant_shifts_lse_only():
    """softmax is invariant to a per-row constant: O unchanged, lse moves by it."""
    q, k, v = _case(1, 2, 1, 4, 6, 4, 3, seed=401)
    base = _add_mask((2, 4, 6), 11)
    shift = np.array([0.5, -3.0, 7.25, 0.0])[None, :, None]
    o1, l1 = sdpa_ref(q, k, v, 0.8, "none", mask_arr=base)
    o2, l2 = sdpa_ref(q, k, v, 0.8, "none", mask_arr=base + shift)
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2 - l1, np.broadcast_to(shift[..., 0], l1.shape), atol=1e-13)


def test_additive_log_weights_closed_form():
    """Adding ln w_j to the scores weights key j by w_j: o = sum w e^s v / sum w e^s."""
    q, k, v = _case(1, 1, 1, 2, 3, 4, 2, seed=411)
    wts = np.array([0.25, 2.0, 5.0])
    o, lse = sdpa_ref(q, k, v, 0.7, "none", mask_arr=np.log(wts))
    for i in range(2):
        e = [wts[j] * math.exp(0.7 * float(q[0, 0, i] @ k[0, 0, j])) for j in range(3)]
        exp = sum(e[j] * v[0, 0, j] for j in range(3)) / sum(e)
        np.testing.assert_allclose(o[0, 0, i], exp, atol=1e-14)
        assert abs(lse[0, 0, i] - math.log(sum(e))) < 1e-13


def test_boolean_and_additive_minus_inf_agree():
    q, k, v = _case(2, 2, 1, 5, 7, 3, 3, seed=421)
    keep = _bool_mask((5, 7), 13)
    keep[:, 0] = True
    o1, l1 = sdpa_ref(q, k, v, 0.5, "causal", mask_arr=keep)
    o2, l2 = sdpa_ref(q, k, v, 0.5, "causal", mask_arr=np.where(keep, 0.0, -np.inf))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_all_true_and_zero_masks_equal_no_mask():
    q, k, v = _case(1, 4, 2, 3, 6, 4, 4, seed=431)
    o, lse = sdpa_ref(q, k, v, 0.5, "window", 2)
    for arr in (np.ones((3, 6), dtype=bool), np.zeros((1, 1, 3, 6))):
        o2, l2 = sdpa_ref(q, k, v, 0.5, "window", 2, mask_arr=arr)
        np.testing.assert_array_equal(o, o2)
        np.testing.assert_array_equal(lse, l2)


def test_boolean_mask_of_the_mode_rule_equals_the_mode():
    """An explicit [Lq, Lk] window array (how callers express a window without
    the window mode) gives the window mode's result."""
    q, k, v = _case(1, 2, 1, 6, 9, 4, 4, seed=441)
    o, lse = sdpa_ref(q, k, v, 0.5, "window", 3)
    o2, l2 = sdpa_ref(q, k, v, 0.5, "none", mask_arr=visible_mask(6, 9, "window", 3))
    np.testing.assert_allclose(o, o2, atol=1e-15)
    np.testing.assert_allclose(lse, l2, atol=1e-15)


def test_single_kept_key_closed_form():
    q, k, v = _case(1, 1, 1, 3, 5, 4, 3, seed=451)
    arr = np.zeros((3, 5), dtype=bool)
    arr[0, 4] = arr[1, 0] = arr[2, 2] = True
    o, lse = sdpa_ref(q, k, v, 0.9, "none", mask_arr=arr)
    for i, j in enumerate([4, 0, 2]):
        np.testing.assert_array_equal(o[0, 0, i], v[0, 0, j])
        assert abs(lse[0, 0, i] - 0.9 * float(q[0, 0, i] @ k[0, 0, j])) < 1e-14


@pytest.mark.parametrize("kind", ["bool", "add"])
def test_empty_rows_give_zero_output_and_minus_inf_lse(kind):
    q, k, v = _case(1, 2, 1, 4, 5, 3, 3, seed=461)
    keep = np.ones((2, 4, 5), dtype=bool)
    keep[0, 1] = False
    keep[1, 3] = False
    arr = keep if kind == "bool" else np.where(keep, 0.5, -np.inf)
    o, lse = sdpa_ref(q, k, v, 0.5, "none", mask_arr=arr)
    for h, i in [(0, 1), (1, 3)]:
        np.testing.assert_array_equal(o[0, h, i], 0.0)
        assert lse[0, h, i] == -math.inf
    o2, l2 = sdpa_loop(q, k, v, 0.5, "none", mask_arr=arr)
    np.testing.assert_array_equal(o2[0, 0, 1], 0.0)
    assert l2[0, 1, 3] == -math.inf
    p = sdpa_probs(q, k, 0.5, "none", mask_arr=arr)
    np.testing.assert_array_equal(p[0, 0, 1], 0.0)
    np.testing.assert_allclose(p[0, 0, 0].sum(), 1.0, atol=1e-15)
    orow, lrow = sdpa_ref_rows(q, k, v, 0.5, "none", 0, [(0, 0, 1), (0, 1, 2)], mask_arr=arr)
    np.testing.assert_array_equal(orow[0], 0.0)
    assert lrow[0] == -math.inf
    np.testing.assert_allclose(orow[1], o[0, 1, 2], atol=1e-14)


def test_per_head_masks_follow_query_heads_not_kv_heads():
    """With GQA a [B, Hq, ...] mask is indexed by the query head: each head's
    result equals a one-head run with that head's slice."""
    q, k, v = _case(1, 4, 2, 3, 6, 4, 4, seed=471)
    arr = _add_mask((1, 4, 3, 6), 17)
    arr[..., 0] = 0.0
    o, lse = sdpa_ref(q, k, v, 0.5, "none", mask_arr=arr)
    for h in range(4):
        o1, l1 = sdpa_ref(q[:, h:h + 1], k[:, h // 2:h // 2 + 1], v[:, h // 2:h // 2 + 1], 0.5, "none",
                          mask_arr=arr[:, h:h + 1])
        np.testing.assert_array_equal(o[:, h:h + 1], o1)
        np.testing.assert_array_equal(lse[:, h:h + 1], l1)


def test_mask_rows_accessor_reads_torch_broadcast_views():
    q, k, v = _case(2, 2, 1, 3, 5, 4, 4, seed=481)
    arr = torch.from_numpy(_add_mask((2, 1, 1, 5), 19)).to(torch.bfloat16)
    o, lse = sdpa_ref(q, k, v, 0.5, "none", mask_arr=arr)
    picks = list(itertools.product(range(2), range(2), range(3)))
    orow, lrow = sdpa_ref_rows(q, k, v, 0.5, "none", 0, picks, mask_arr=arr)
    for n, (bi, h, i) in enumerate(picks):
        np.testing.assert_allclose(orow[n], o[bi, h, i], atol=1e-13)
        assert abs(lrow[n] - lse[bi, h, i]) < 1e-13


def test_bad_additive_values_raise():
    q, k, v = _case(1, 1, 1, 2, 3, 2, 2, seed=491)
    for bad in (np.inf, np.nan):
        arr = np.zeros((2, 3))
        arr[1, 1] = bad
        with pytest.raises(ValueError):
            sdpa_ref(q, k, v, 0.5, "none", mask_arr=arr)


# ---------------------------------------------------------------------------
# Per-batch lengths (varlen): batch entry b uses its first q_lens[b] queries
# and kv_lens[b] keys, query i at key position i + kv_lens[b] - q_lens[b].
# ---------------------------------------------------------------------------

from oracle import sdpa_ref_varlen, visible_offset  # noqa: E402

VARLEN = [
    # b, hq, hkv, lq, lk, dqk, dv, mode, window, q_lens, kv_lens
    (3, 2, 1, 4, 7, 3, 4, "none", 0, [4, 2, 1], [7, 3, 0]),
    (3, 4, 2, 5, 8, 4, 3, "causal", 0, [5, 3, 4], [8, 5, 2]),
    (2, 2, 2, 6, 9, 3, 3, "window", 3, [6, 2], [9, 4]),
    (2, 2, 1, 3, 6, 2, 2, "causal", 0, [3, 1], [6, 6]),
]


@pytest.mark.parametrize("case", VARLEN)
def test_varlen_matches_loop_brute_force(case):
    b, hq, hkv, lq, lk, dqk, dv, mode, w, ql, kl = case
    q, k, v = _case(b, hq, hkv, lq, lk, dqk, dv, seed=600 + lq)
    o, lse = sdpa_ref_varlen(q, k, v, 0.7, mode, w, ql, kl)
    o2, l2 = sdpa_loop(q, k, v, 0.7, mode, w, q_lens=ql, kv_lens=kl)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)  # NaN rows (past q_lens) match too
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)
    for bi in range(b):
        assert np.isnan(o[bi, :, ql[bi]:]).all() and not np.isnan(o[bi, :, :ql[bi]]).any()


@pytest.mark.parametrize("case", VARLEN)
def test_varlen_entry_equals_the_unpadded_problem(case):
    """Each entry with q_lens <= kv_lens equals the plain definition on its
    valid slices (bottom-right aligned), and padding keys never matter."""
    b, hq, hkv, lq, lk, dqk, dv, mode, w, ql, kl = case
    q, k, v = _case(b, hq, hkv, lq, lk, dqk, dv, seed=610 + lq)
    o, lse = sdpa_ref_varlen(q, k, v, 0.5, mode, w, ql, kl)
    k2, v2 = k.copy(), v.copy()
    for bi in range(b):
        k2[bi, :, kl[bi]:] = 1e3
        v2[bi, :, kl[bi]:] = -1e3
        if 0 < ql[bi] <= kl[bi]:
            so, sl = sdpa_ref(q[bi:bi + 1, :, :ql[bi]], k[bi:bi + 1, :, :kl[bi]], v[bi:bi + 1, :, :kl[bi]],
                              0.5, mode, w)
            np.testing.assert_allclose(o[bi:bi + 1, :, :ql[bi]], so, atol=1e-14)
            np.testing.assert_allclose(lse[bi:bi + 1, :, :ql[bi]], sl, atol=1e-14)
    o2, l2 = sdpa_ref_varlen(q, k2, v2, 0.5, mode, w, ql, kl)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(l2, lse)


def test_varlen_matches_torch_cpu_sdpa():
    """torch's float64 attention per entry, with an explicit boolean mask over
    the padded key range written out here from the length rule."""
    b, hq, hkv, lq, lk, d = 3, 4, 2, 5, 9, 4
    ql, kl = [5, 4, 2], [9, 6, 7]
    q, k, v = _case(b, hq, hkv, lq, lk, d, d, seed=620)
    o, _ = sdpa_ref_varlen(q, k, v, 0.45, "window", 3, ql, kl)
    for bi in range(b):
        m = np.zeros((lq, lk), dtype=bool)
        for i in range(ql[bi]):
            p = i + kl[bi] - ql[bi]
            for j in range(kl[bi]):
                m[i, j] = p - 3 < j <= p
        got = _torch_sdpa(q[bi:bi + 1, :, :ql[bi]], k[bi:bi + 1], v[bi:bi + 1], 0.45, m[:ql[bi]])
        np.testing.assert_allclose(o[bi:bi + 1, :, :ql[bi]], got, atol=1e-12)


def test_varlen_empty_entries_and_rows_before_the_first_key():
    q, k, v = _case(2, 2, 1, 4, 5, 3, 3, seed=630)
    # entry 0: no keys at all; entry 1: causal, 4 queries on 2 keys -> the
    # first two rows sit before key 0 and see nothing
    o, lse = sdpa_ref_varlen(q, k, v, 0.5, "causal", 0, [3, 4], [0, 2])
    np.testing.assert_array_equal(o[0, :, :3], 0.0)
    assert np.isneginf(lse[0, :, :3]).all()
    np.testing.assert_array_equal(o[1, :, :2], 0.0)
    assert np.isneginf(lse[1, :, :2]).all()
    np.testing.assert_allclose(o[1, 0, 2], v[1, 0, 0], atol=1e-15)  # row 2 sees key 0 only
    assert abs(lse[1, 0, 2] - 0.5 * float(q[1, 0, 2] @ k[1, 0, 0])) < 1e-14


def test_varlen_rows_accessor_agrees():
    q, k, v = _case(2, 4, 2, 6, 9, 4, 4, seed=640)
    ql, kl = [6, 3], [9, 5]
    arr = _add_mask((2, 1, 6, 9), 23)
    arr[..., 0] = 0.0
    o, lse = sdpa_ref_varlen(q, k, v, 0.5, "causal", 0, ql, kl, mask_arr=arr)
    picks = [(bi, h, i) for bi in range(2) for h in range(4) for i in range(ql[bi])]
    orow, lrow = sdpa_ref_rows(q, k, v, 0.5, "causal", 0, picks, mask_arr=arr, q_lens=ql, kv_lens=kl)
    for n, (bi, h, i) in enumerate(picks):
        np.testing.assert_allclose(orow[n], o[bi, h, i], atol=1e-13)
        assert (np.isneginf(lrow[n]) and np.isneginf(lse[bi, h, i])) or abs(lrow[n] - lse[bi, h, i]) < 1e-13


def test_visible_offset_generalises_bottom_right():
    for lq, lk, mode, w in [(4, 9, "causal", 0), (9, 9, "window", 3), (3, 3, "none", 0)]:
        np.testing.assert_array_equal(visible_offset(lq, lk, lk - lq, mode, w), visible_mask(lq, lk, mode, w))
    assert not visible_offset(3, 4, -3, "causal").any()  # every row before key 0
    np.testing.assert_array_equal(visible_offset(2, 4, 1, "causal"), [[1, 1, 0, 0], [1, 1, 1, 0]])


def test_bad_lengths_raise():
    q, k, v = _case(2, 1, 1, 3, 4, 2, 2, seed=650)
    for ql, kl in [([3, 4], [4, 4]), ([3, 3], [5, 4]), ([3, -1], [4, 4]), ([3], [4])]:
        with pytest.raises(ValueError):
            sdpa_ref_varlen(q, k, v, 0.5, "none", 0, ql, kl)
