"""Pins for the float64 backward oracle (no GPU): torch's float64 autograd
through its CPU attention (library special case), central finite differences
of the forward oracle, and exact invariants of the gradient formulas."""

import numpy as np
import pytest
import torch

from oracle import sdpa_bwd_ref, sdpa_bwd_ref_varlen, sdpa_ref, sdpa_ref_varlen, visible_mask


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(b, hq, hkv, lq, lk, dqk, dv, seed):
    return (_rand((b, hq, lq, dqk), seed), _rand((b, hkv, lk, dqk), seed + 1),
            _rand((b, hkv, lk, dv), seed + 2), _rand((b, hq, lq, dv), seed + 3))


CASES = [
    # b, hq, hkv, lq, lk, dqk, dv, mask, window
    (1, 2, 2, 4, 6, 3, 5, "none", 0),
    (2, 4, 2, 5, 5, 4, 4, "causal", 0),
    (1, 4, 1, 3, 8, 5, 3, "causal", 0),
    (1, 2, 1, 6, 9, 4, 2, "window", 3),
]


@pytest.mark.parametrize("case", CASES)
def test_bwd_matches_torch_autograd(case):
    b, hq, hkv, lq, lk, dqk, dv, mask, w = case
    q, k, v, do = _case(b, hq, hkv, lq, lk, dqk, dv, seed=700 + lq)
    dq, dk, dvv = sdpa_bwd_ref(q, k, v, do, 0.6, mask, w)
    g = hq // hkv
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    m = torch.from_numpy(visible_mask(lq, lk, mask, w))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=m, scale=0.6)
    out.backward(torch.from_numpy(do))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dvv, tv.grad.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("case", CASES[1:3])
def test_bwd_matches_finite_differences(case):
    """dL/dx for L = sum(O * dO), central differences of the forward oracle."""
    b, hq, hkv, lq, lk, dqk, dv, mask, w = case
    q, k, v, do = _case(b, hq, hkv, lq, lk, dqk, dv, seed=710 + lq)
    grads = sdpa_bwd_ref(q, k, v, do, 0.8, mask, w)
    rng = np.random.default_rng(3)
    h = 1e-6

    def loss(qq, kk, vv):
        return float((sdpa_ref(qq, kk, vv, 0.8, mask, w)[0] * do).sum())

    for which, x in enumerate((q, k, v)):
        for _ in range(6):
            idx = tuple(int(rng.integers(n)) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grads[which][idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grads[which][idx])


@pytest.mark.parametrize("case", CASES)
def test_bwd_invariants(case):
    """Rows of dS sum to 0, so the keys' dK sum to 0; rows of P sum to 1, so
    the keys' dV sum to the group's summed dO."""
    b, hq, hkv, lq, lk, dqk, dv, mask, w = case
    q, k, v, do = _case(b, hq, hkv, lq, lk, dqk, dv, seed=720 + lq)
    _, dk, dvv = sdpa_bwd_ref(q, k, v, do, 0.7, mask, w)
    g = hq // hkv
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    for kvh in range(hkv):
        np.testing.assert_allclose(dvv[:, kvh].sum(axis=1), do[:, kvh * g:(kvh + 1) * g].sum(axis=(1, 2)),
                                   atol=1e-12)


def test_bwd_unseen_keys_get_no_gradient():
    q, k, v, do = _case(1, 2, 1, 3, 10, 4, 4, seed=730)
    _, dk, dvv = sdpa_bwd_ref(q, k, v, do, 0.5, "window", 2)  # rows see keys 6..9 only
    np.testing.assert_array_equal(dk[:, :, :6], 0.0)
    np.testing.assert_array_equal(dvv[:, :, :6], 0.0)
    assert np.abs(dk[:, :, 6:]).sum() > 0 and np.abs(dvv[:, :, 7:]).sum() > 0


def test_bwd_scale_zero():
    q, k, v, do = _case(1, 2, 2, 3, 5, 4, 3, seed=740)
    dq, dk, dvv = sdpa_bwd_ref(q, k, v, do, 0.0, "none")
    np.testing.assert_array_equal(dq, 0.0)
    np.testing.assert_array_equal(dk, 0.0)
    # uniform P = 1/Lk: every key's dV is the rows' summed dO over Lk
    np.testing.assert_allclose(dvv, np.broadcast_to(do.sum(axis=2, keepdims=True) / 5, (1, 2, 5, 3)), atol=1e-15)


def test_bwd_single_key_closed_form():
    """One key: P = 1, dV = sum of dO over the rows, dS = 0 so dQ = dK = 0."""
    q, k, v, do = _case(1, 2, 1, 3, 1, 4, 3, seed=750)
    dq, dk, dvv = sdpa_bwd_ref(q, k, v, do, 0.9, "none")
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dvv[0, 0, 0], do[0].sum(axis=(0, 1)), atol=1e-14)


# ---- per-batch lengths ----

VARLEN = [
    # b, hq, hkv, lq, lk, dqk, dv, mask, window, q_lens, kv_lens
    (3, 4, 2, 5, 7, 3, 4, "causal", 0, [5, 2, 3], [7, 3, 0]),
    (2, 2, 1, 4, 6, 4, 3, "none", 0, [4, 1], [2, 6]),
    (2, 2, 2, 6, 8, 3, 3, "window", 3, [6, 4], [8, 5]),
    (2, 4, 2, 4, 5, 2, 2, "causal", 0, [4, 3], [2, 5]),  # entry 0: more queries than keys
]


def test_bwd_varlen_full_lengths_is_the_dense_gradient():
    q, k, v, do = _case(2, 4, 2, 5, 7, 3, 4, seed=730)
    a = sdpa_bwd_ref(q, k, v, do, 0.7, "causal", 0)
    c = sdpa_bwd_ref_varlen(q, k, v, do, 0.7, "causal", 0, [5, 5], [7, 7])
    for x, y in zip(a, c):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("case", VARLEN)
def test_bwd_varlen_matches_finite_differences(case):
    """dL/dx for L = sum over the valid output rows of O * dO, by central
    differences of the forward's per-length oracle; every position past the
    lengths has gradient 0."""
    b, hq, hkv, lq, lk, dqk, dv, mask, w, ql, kl = case
    q, k, v, do = _case(b, hq, hkv, lq, lk, dqk, dv, seed=740 + lq)
    grads = sdpa_bwd_ref_varlen(q, k, v, do, 0.9, mask, w, ql, kl)
    h = 1e-6

    def loss(qq, kk, vv):
        o, _ = sdpa_ref_varlen(qq, kk, vv, 0.9, mask, w, ql, kl)
        return float(np.nansum(o * do))

    for which, x in enumerate((q, k, v)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grads[which][idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grads[which][idx])


def test_bwd_varlen_rows_without_keys():
    """A causal entry with more queries than keys: its first rows see no key,
    output the constant 0 and take no gradient; keys past kv_lens get none."""
    q, k, v, do = _case(1, 2, 1, 4, 6, 3, 3, seed=760)
    dq, dk, dv = sdpa_bwd_ref_varlen(q, k, v, do, 0.5, "causal", 0, [4], [2])
    assert (dq[0, :, :2] == 0).all() and np.abs(dq[0, :, 2:]).max() > 0
    assert (dk[0, :, 2:] == 0).all() and (dv[0, :, 2:] == 0).all()


# ---- explicit mask arrays ----

def test_bwd_mask_arrays_match_torch_autograd():
    """Boolean and additive mask arrays (broadcast over heads), through
    torch's float64 autograd with the combined mask written out."""
    b, hq, hkv, lq, lk, d = 2, 4, 2, 5, 7, 3
    q, k, v, do = _case(b, hq, hkv, lq, lk, d, d, seed=780)
    rng = np.random.default_rng(781)
    keep = rng.random((b, 1, lq, lk)) < 0.7
    keep[..., 0] = True  # key 0 is visible to every row under causal (Lk > Lq): no row is left empty
    vis = visible_mask(lq, lk, "causal", 0)
    add = rng.standard_normal((1, hq, lq, lk))
    g = hq // hkv
    for arr, tmask in ((keep, torch.from_numpy(np.broadcast_to(keep, (b, hq, lq, lk)) & vis)),
                       (add, torch.from_numpy(np.where(vis, np.broadcast_to(add, (b, hq, lq, lk)), -np.inf)))):
        dq, dk, dvv = sdpa_bwd_ref(q, k, v, do, 0.6, "causal", 0, mask_arr=arr)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(g, dim=1), tv.repeat_interleave(g, dim=1), attn_mask=tmask, scale=0.6)
        out.backward(torch.from_numpy(do))
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dvv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_bwd_varlen_mask_array_matches_finite_differences():
    """Per-batch lengths with a boolean array that removes every key of one
    row (that row's output is the constant 0): central differences of the
    per-length forward oracle, every element."""
    b, hq, hkv, lq, lk, d = 2, 2, 1, 4, 5, 2
    q, k, v, do = _case(b, hq, hkv, lq, lk, d, d, seed=790)
    keep = np.random.default_rng(791).random((b, hq, lq, lk)) < 0.6
    keep[0, 1, 2, :] = False
    ql, kl = [4, 3], [5, 4]
    grads = sdpa_bwd_ref_varlen(q, k, v, do, 0.7, "none", 0, ql, kl, mask_arr=keep)
    h = 1e-6

    def loss(qq, kk, vv):
        o, _ = sdpa_ref_varlen(qq, kk, vv, 0.7, "none", 0, ql, kl, mask_arr=keep)
        return float(np.nansum(o * do))

    for which, x in enumerate((q, k, v)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grads[which][idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grads[which][idx])
    assert (grads[0][0, 1, 2] == 0).all()
