"""GPU parity of the fused forward against the float64 oracle, whole outputs.

Sizes are small enough for the oracle to finish in seconds but span several
row tiles and key blocks with ragged tails.  Every case prints its parameters
before touching the GPU.
"""

import zlib

import numpy as np
import pytest
import torch

import scaled_dot_product_fwd_amd as sdpa
from gpu_cases import TOL_O, check_full, run_gpu
from scaled_dot_product_fwd_amd.synth import default_scale, make_qkv

pytestmark = pytest.mark.gpu


def _say(*a):
    print("CASE", *a, flush=True)


def test_tiny_fp32_config():
    """B=1, Hq=Hkv=4, Lq=Lk=128, D=64, float32, no mask, scale 1/sqrt(64)."""
    _say("tiny fp32 config")
    check_full(1, 4, 4, 128, 128, 64, 64, "f32", "none", 0, seed=1000)


CASES = [
    # b, hq, hkv, lq, lk, dqk, dv, dtype, mask, window
    (1, 4, 2, 200, 200, 64, 64, "bf16", "causal", 0),
    (2, 4, 1, 77, 300, 128, 128, "f16", "causal", 0),
    (1, 2, 2, 300, 300, 72, 72, "bf16", "none", 0),
    (1, 2, 1, 150, 333, 96, 96, "bf16", "window", 37),
    (1, 2, 2, 257, 257, 8, 8, "bf16", "none", 0),
    (1, 2, 2, 130, 130, 80, 80, "f16", "causal", 0),
    (1, 2, 1, 140, 140, 256, 256, "bf16", "causal", 0),
    (1, 2, 2, 129, 129, 160, 160, "f16", "window", 64),
    (1, 2, 2, 100, 100, 224, 224, "bf16", "none", 0),
    (1, 32, 2, 1, 1000, 192, 128, "bf16", "none", 0),
    (1, 16, 1, 3, 777, 192, 128, "bf16", "causal", 0),
    (1, 8, 8, 5, 400, 192, 192, "f16", "causal", 0),
    (1, 4, 1, 12, 2000, 128, 128, "f16", "none", 0),
    (1, 4, 1, 8, 2000, 128, 128, "f16", "none", 0),
    (1, 4, 1, 24, 1500, 128, 128, "f16", "causal", 0),
    (1, 4, 2, 64, 64, 64, 64, "f32", "causal", 0),
    (2, 4, 2, 70, 190, 128, 128, "f32", "window", 50),
    (1, 4, 4, 33, 33, 96, 96, "f32", "none", 0),
    (1, 8, 2, 1, 4096, 32, 64, "f32", "none", 0),
    (1, 3, 1, 40, 500, 64, 32, "bf16", "none", 0),
    (1, 2, 2, 96, 96, 16, 48, "f16", "causal", 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) for x in c))
def test_small_cases(case):
    b, hq, hkv, lq, lk, dqk, dv, dt, mask, w = case
    _say(case)
    check_full(b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, seed=zlib.crc32(repr(case).encode()) % 10000)


@pytest.mark.parametrize("lk", [1, 2, 63, 64, 65, 127, 129])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_short_key_lengths(lk, dt):
    _say("short lk", lk, dt)
    check_full(1, 4, 2, 1, lk, 64, 64, dt, "none", 0, seed=lk)
    lq = min(lk, 5)
    check_full(1, 4, 2, lq, lk, 64, 64, dt, "causal", 0, seed=lk + 1)


@pytest.mark.parametrize("w", [1, 2, 63, 64, 65, 127, 128, 129, 1000])
def test_window_edges(w):
    """Unaligned and aligned window edges, including a window of one key."""
    _say("window", w)
    check_full(1, 2, 1, 260, 300, 64, 64, "bf16", "window", w, seed=w)


def test_window_1000_unaligned_prefill():
    """A window whose lower edge is not block aligned (W=1000) over several tiles."""
    _say("window 1000 prefill")
    check_full(1, 2, 2, 2100, 2100, 64, 64, "bf16", "window", 1000, seed=5)


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 8, 16])
def test_forced_splits_agree(splits):
    _say("splits", splits)
    check_full(1, 8, 2, 4, 3000, 128, 128, "bf16", "causal", 0, seed=77, num_splits=splits)


@pytest.mark.parametrize("row_tile", [32, 64, 128])
@pytest.mark.parametrize("mask,w", [("none", 0), ("causal", 0), ("window", 100)])
def test_forced_row_tiles_agree(row_tile, mask, w):
    _say("row tile", row_tile, mask, w)
    check_full(1, 4, 2, 90, 700, 64, 64, "f16", mask, w, seed=row_tile, row_tile=row_tile)


def test_strided_kv_cache_view():
    """K/V are views into a cache with capacity beyond Lk (non-contiguous head stride)."""
    _say("strided kv cache")
    from oracle import sdpa_ref
    cap, lk, lq = 512, 300, 7
    q, kc, vc = make_qkv(1, 8, 2, lq, cap, 128, 128, torch.bfloat16, 42)
    k, v = kc[:, :, :lk], vc[:, :, :lk]
    dev = torch.device("cuda", 0)
    kd, vd = kc.to(dev)[:, :, :lk], vc.to(dev)[:, :, :lk]
    assert not kd.is_contiguous()
    o, lse = sdpa.forward(q.to(dev), kd, vd, mask="causal", return_lse=True)
    ro, rl = sdpa_ref(q, k, v, default_scale(128), "causal", 0)
    assert float(np.abs(o.double().cpu().numpy() - ro).max()) <= TOL_O[torch.bfloat16]
    assert float(np.abs(lse.double().cpu().numpy() - rl).max()) <= 1e-4


def test_batch_two_gqa_eight():
    _say("batch 2, G=8")
    check_full(2, 16, 2, 33, 257, 64, 64, "bf16", "causal", 0, seed=9)


def test_large_magnitude_queries_stay_finite():
    _say("large q")
    q, k, v = make_qkv(1, 4, 2, 64, 500, 64, 64, torch.bfloat16, 3)
    q = (q.float() * 30).to(torch.bfloat16)
    o, lse = run_gpu(q, k, v, default_scale(64), "causal", 0)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    from oracle import sdpa_ref
    ro, rl = sdpa_ref(q, k, v, default_scale(64), "causal", 0)
    assert float(np.abs(o - ro).max()) <= 2e-2
    assert float(np.abs(lse - rl).max() / max(1.0, np.abs(rl).max())) <= 1e-5


def test_monotone_scores_running_max_changes_every_block():
    """Keys ordered so the running max rises (then falls) block after block."""
    _say("monotone scores")
    from oracle import sdpa_ref
    lk, d = 1024, 64
    q = torch.ones(1, 1, 2, d)
    ramp = torch.linspace(-4, 4, lk)[:, None].repeat(1, d) / d
    for sign in (1.0, -1.0):
        k = (sign * ramp)[None, None].to(torch.float16)
        v = torch.randn(1, 1, lk, d, generator=torch.Generator().manual_seed(1)).to(torch.float16)
        qq = q.to(torch.float16)
        o, lse = run_gpu(qq, k, v, 1.0, "none", 0)
        ro, rl = sdpa_ref(qq, k, v, 1.0, "none", 0)
        assert float(np.abs(o - ro).max()) <= 5e-3
        assert float(np.abs(lse - rl).max()) <= 1e-4


@pytest.mark.parametrize("d", [192, 224, 256])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_large_head_dims_every_block_count(d, dt):
    """Prefill tiles at head dims 192-256 run 32-key blocks through a fixed
    product order, two blocks per loop turn: one to six blocks (either parity
    of the pair loop, a ragged last block), unmasked, causal and windowed,
    three 128-row tiles with a ragged last one."""
    for lk in (20, 64, 90, 128, 150, 190):
        _say("large dims", d, dt, lk)
        check_full(1, 2, 1, 130, lk, d, d, dt, "none", 0, seed=lk + d)
        lq = min(lk, 130)
        check_full(1, 2, 1, lq, lk, d, d, dt, "causal", 0, seed=lk + d + 1)
        check_full(1, 2, 1, lq, lk, d, d, dt, "window", 40, seed=lk + d + 2)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_monotone_scores_large_head_dim_prefill(dt):
    """The running max rises (then falls) block after block in 128-row tiles
    at head dim 256, so the rescale of O between the matrix products runs."""
    _say("monotone scores D256", dt)
    from oracle import sdpa_ref
    lk, d = 700, 256
    q = torch.ones(1, 1, 130, d)
    # scores -40 .. 40: the block max climbs by more than the lazy-rescale
    # threshold block after block
    ramp = torch.linspace(-40, 40, lk)[:, None].repeat(1, d) / d
    for sign in (1.0, -1.0):
        k = (sign * ramp)[None, None].to(dt)
        v = torch.randn(1, 1, lk, d, generator=torch.Generator().manual_seed(2)).to(dt)
        qq = q.to(dt)
        o, lse = run_gpu(qq, k, v, 1.0, "none", 0)
        ro, rl = sdpa_ref(qq, k, v, 1.0, "none", 0)
        assert float(np.abs(o - ro).max()) <= TOL_O[dt]
        assert float(np.abs(lse - rl).max()) <= 1e-4


def test_single_spike_key_in_last_split():
    _say("spike in last split")
    from oracle import sdpa_ref
    q, k, v = make_qkv(1, 8, 1, 1, 4000, 128, 128, torch.bfloat16, 11)
    k[0, 0, 3990] = (q[0, 0, 0].float() * 3).to(torch.bfloat16)
    o, lse = run_gpu(q, k, v, default_scale(128), "none", 0, num_splits=8)
    ro, rl = sdpa_ref(q, k, v, default_scale(128), "none", 0)
    assert float(np.abs(o - ro).max()) <= 2e-2
    assert float(np.abs(lse - rl).max()) <= 1e-4


def test_fixed_plan_is_bitwise_deterministic():
    _say("determinism")
    q, k, v = make_qkv(1, 8, 2, 16, 3000, 128, 128, torch.bfloat16, 21)
    a = run_gpu(q, k, v, default_scale(128), "none", 0)
    b = run_gpu(q, k, v, default_scale(128), "none", 0)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_negative_and_zero_scale():
    _say("scale sign")
    from oracle import sdpa_ref
    q, k, v = make_qkv(1, 2, 1, 20, 200, 64, 64, torch.float16, 31)
    for scale in (-0.3, 0.0):
        o, lse = run_gpu(q, k, v, scale, "causal", 0)
        ro, rl = sdpa_ref(q, k, v, scale, "causal", 0)
        assert float(np.abs(o - ro).max()) <= 5e-3
        assert float(np.abs(lse - rl).max()) <= 1e-4


def test_output_without_lse():
    _say("no lse")
    q, k, v = make_qkv(1, 4, 4, 50, 60, 64, 64, torch.bfloat16, 2)
    dev = torch.device("cuda", 0)
    o = sdpa.forward(q.to(dev), k.to(dev), v.to(dev), mask="causal")
    from oracle import sdpa_ref
    ro, _ = sdpa_ref(q, k, v, default_scale(64), "causal", 0)
    assert float(np.abs(o.double().cpu().numpy() - ro).max()) <= 2e-2


def test_error_leaves_output_untouched():
    _say("error path")
    dev = torch.device("cuda", 0)
    q = torch.randn(1, 2, 9, 64, device=dev, dtype=torch.bfloat16)
    k = torch.randn(1, 2, 8, 64, device=dev, dtype=torch.bfloat16)
    out = torch.full((1, 2, 9, 64), 7.0, device=dev, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="Lq <= Lk"):
        sdpa.forward(q, k, k, mask="causal", out=out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_split_workspace_reused_across_calls():
    """One caller workspace serves split plans of different shapes in a row."""
    from oracle import sdpa_ref
    dev = torch.device("cuda", 0)
    cases = [(1, 8, 2, 4, 3000, 128, 128, 8), (2, 16, 4, 1, 5000, 64, 64, 16),
             (1, 8, 2, 4, 3000, 128, 128, 3), (1, 4, 1, 40, 2100, 192, 128, 5)]
    need = 0
    for b, hq, hkv, lq, lk, dqk, dv, sp in cases:
        d = sdpa.make_desc((b, hq, lq, dqk), (b, hkv, lk, dqk), (b, hkv, lk, dv), sdpa.SDPA_BF16,
                           mask="causal", num_splits=sp)
        need = max(need, sdpa.sdpa_workspace_bytes(d))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    for rep in range(2):
        for n, (b, hq, hkv, lq, lk, dqk, dv, sp) in enumerate(cases):
            _say("shared workspace", rep, n, b, hq, hkv, lq, lk, dqk, dv, "splits", sp)
            q, k, v = make_qkv(b, hq, hkv, lq, lk, dqk, dv, torch.bfloat16, 90 + n)
            o, lse = sdpa.forward(q.to(dev), k.to(dev), v.to(dev), mask="causal", return_lse=True,
                                  num_splits=sp, workspace=ws)
            torch.cuda.synchronize()
            ro, rl = sdpa_ref(q, k, v, default_scale(dqk), "causal", 0)
            assert float(np.abs(o.double().cpu().numpy() - ro).max()) <= TOL_O[torch.bfloat16]
            assert float(np.abs(lse.double().cpu().numpy() - rl).max()) <= 1e-4


@pytest.mark.parametrize("splits", [7, 16])
def test_more_splits_than_key_blocks(splits):
    """Splits left without any key block publish m = -inf, l = 0 and must
    drop out of the merge."""
    _say("empty splits", splits)
    check_full(1, 4, 1, 2, 150, 64, 64, "f16", "none", 0, seed=55, num_splits=splits)


@pytest.mark.parametrize("lq", [96, 130])
def test_split_plan_with_several_row_tiles(lq):
    """Split plans with more than one row tile per KV head deal their work
    items to XCDs in groups; every row must still come out exactly once."""
    _say("split + row tiles", lq)
    d = sdpa.make_desc((1, 32, lq, 128), (1, 8, 3000, 128), (1, 8, 3000, 128), sdpa.SDPA_F16)
    plan = dict(t.split("=", 1) for t in sdpa.sdpa_describe_plan(d).split())
    assert int(plan["row_tiles"]) > 1 and int(plan["splits"]) > 1 and plan["xcd_group"] == "8"
    check_full(1, 32, 8, lq, 3000, 128, 128, "f16", "none", 0, seed=61)


@pytest.mark.parametrize("b,hkv,lq", [(1, 8, 1), (2, 8, 2), (3, 8, 3)])
def test_split_heads_grouped_by_xcd(b, hkv, lq):
    """One row tile per KV head and B Hkv a multiple of 8: each head's splits
    and its combine rows are dealt to one XCD (8, 16 and 24 head rows, so
    one to three groups of eight); every row must come out exactly once."""
    _say("split heads by XCD", b, hkv, lq)
    d = sdpa.make_desc((b, 4 * hkv, lq, 128), (b, hkv, 2500, 128), (b, hkv, 2500, 128), sdpa.SDPA_BF16,
                       mask="causal")
    plan = dict(t.split("=", 1) for t in sdpa.sdpa_describe_plan(d).split())
    assert plan["row_tiles"] == "1" and int(plan["splits"]) > 1 and plan["combine_xcd"] == "1"
    assert plan["xcd_group"] == plan["splits"]
    check_full(b, 4 * hkv, hkv, lq, 2500, 128, 128, "bf16", "causal", 0, seed=67 + b)


HEAD_DIM_80 = [
    # b, hq, hkv, lq, lk, dqk, dv, dtype, mask, window, family, forced plan
    (1, 16, 4, 1, 777, 72, 72, "bf16", "none", 0, "decode", {}),
    (1, 16, 2, 3, 1000, 80, 80, "f16", "causal", 0, "decode", {}),
    (1, 8, 2, 12, 1500, 72, 72, "bf16", "causal", 0, "short", {}),
    (1, 16, 2, 40, 900, 80, 80, "bf16", "none", 0, "prefill", {}),
    (1, 32, 8, 48, 700, 72, 64, "f16", "window", 100, "wide", {}),
    (2, 2, 2, 300, 300, 72, 72, "f16", "none", 0, "prefill", {}),
    (2, 2, 2, 300, 300, 72, 72, "bf16", "causal", 0, "prefill", {"num_splits": 1}),
    (1, 2, 1, 333, 333, 80, 96, "bf16", "causal", 0, "prefill", {}),
    (1, 3, 1, 200, 450, 64, 96, "bf16", "window", 77, "prefill", {"num_splits": 1}),
    (1, 4, 2, 190, 260, 72, 72, "f16", "window", 50, "short", {"row_tile": 64, "num_splits": 1}),
]


@pytest.mark.parametrize("case", HEAD_DIM_80, ids=lambda c: "-".join(str(x) for x in c[:11]))
def test_qk_head_dim_80_every_family(case):
    """Head dims 65-80 take the (80, 96) kernels: Q and K padded to 80 (a
    K row of ten 16-byte chunks, swizzled in pairs), V to 96."""
    b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, fam, plan = case
    _say("qk80", case)
    code = sdpa.SDPA_BF16 if dt == "bf16" else sdpa.SDPA_F16
    d = sdpa.make_desc((b, hq, lq, dqk), (b, hkv, lk, dqk), (b, hkv, lk, dv), code, mask=mask,
                       window_size=w, **plan)
    got = dict(t.split("=", 1) for t in sdpa.sdpa_describe_plan(d).split())
    assert got["family"] == fam and got["dqk"] == f"{dqk}->80" and got["dv"] == f"{dv}->96", got
    check_full(b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, seed=zlib.crc32(repr(case).encode()) % 10000, **plan)


WIDE = [
    # 128 < packed rows <= 256: the wide family (256-row tiles, eight waves)
    (1, 32, 8, 48, 2000, 128, 128, "f16", "none", 0),
    (1, 32, 8, 64, 1500, 128, 128, "bf16", "causal", 0),
    (2, 2, 1, 200, 333, 64, 64, "bf16", "causal", 0),
    (1, 4, 2, 90, 300, 96, 96, "f32", "window", 40),
    (1, 2, 2, 129, 129, 72, 72, "bf16", "none", 0),
    # tiles of five or six 32-row groups (one key block, two, ragged groups,
    # causal, window)
    (1, 32, 8, 48, 20, 128, 128, "bf16", "none", 0),
    (1, 32, 8, 48, 70, 128, 128, "f16", "causal", 0),
    (1, 4, 1, 40, 300, 128, 128, "bf16", "none", 0),
    (1, 4, 1, 37, 333, 128, 128, "f16", "causal", 0),
    (1, 8, 2, 45, 500, 128, 128, "bf16", "window", 100),
    (1, 8, 2, 50, 333, 64, 64, "bf16", "window", 37),
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "-".join(str(x) for x in c))
def test_wide_family(case):
    b, hq, hkv, lq, lk, dqk, dv, dt, mask, w = case
    _say("wide", case)
    check_full(b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, seed=zlib.crc32(repr(case).encode()) % 10000)


def test_wide_family_more_splits_than_blocks():
    # 200 keys in 64-key blocks, 16 splits: some workgroups get one block, some none
    _say("wide, 16 splits over 4 blocks")
    check_full(1, 32, 8, 48, 200, 128, 128, "f16", "none", 0, seed=91, num_splits=16)
    # five row groups with a split key range
    _say("wide, five row groups, 5 splits")
    check_full(1, 4, 1, 40, 900, 128, 128, "bf16", "none", 0, seed=92, num_splits=5)


def test_window_tiles_grouped_by_xcd_full_parity():
    # 2 x 32 KV heads x 16 row tiles = 1024 window workgroups: the plan groups
    # neighbouring tiles on one XCD (xcd_group = 8); every element is checked
    desc = sdpa.make_desc((2, 32, 2048, 32), (2, 32, 2048, 32), (2, 32, 2048, 32), sdpa.SDPA_BF16,
                          mask="window", window_size=300)
    plan = dict(tok.split("=", 1) for tok in sdpa.sdpa_describe_plan(desc).split())
    assert plan["xcd_group"] == "8" and plan["grid"] == "1024", plan
    _say("window tiles grouped by XCD, full parity")
    check_full(2, 32, 32, 2048, 2048, 32, 32, "bf16", "window", 300, seed=93)


def test_unmasked_prefill_tiles_grouped_by_xcd_full_parity():
    # 16 heads x 16 row tiles of 64 rows = 256 workgroups: the tiles of each
    # head run as one group on one XCD (xcd_group = 16); every element is checked
    desc = sdpa.make_desc((1, 16, 1024, 64), (1, 16, 1024, 64), (1, 16, 1024, 64), sdpa.SDPA_BF16)
    plan = dict(tok.split("=", 1) for tok in sdpa.sdpa_describe_plan(desc).split())
    assert plan["xcd_group"] == "16" and plan["grid"] == "256" and plan["splits"] == "1", plan
    _say("unmasked prefill tiles grouped by XCD, full parity")
    check_full(1, 16, 16, 1024, 1024, 64, 64, "bf16", "none", 0, seed=94)
    # 12 heads x 12 tiles of 128 rows in groups of 6 (the encoder arrangement)
    desc = sdpa.make_desc((1, 12, 1500, 64), (1, 12, 1500, 64), (1, 12, 1500, 64), sdpa.SDPA_F16)
    plan = dict(tok.split("=", 1) for tok in sdpa.sdpa_describe_plan(desc).split())
    assert plan["row_tiles"] == "12" and plan["xcd_group"] == "6" and plan["splits"] == "1", plan
    check_full(1, 12, 12, 1500, 1500, 64, 64, "f16", "none", 0, seed=95)


def test_forced_256_row_tiles_on_a_long_prefill():
    _say("row_tile 256 prefill")
    check_full(1, 4, 2, 300, 300, 128, 128, "bf16", "causal", 0, seed=3, row_tile=256)
