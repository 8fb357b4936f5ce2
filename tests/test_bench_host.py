"""Host-side checks of the bench's work accounting (no GPU)."""

import pytest

import bench
from oracle import visible_mask, visible_pairs


@pytest.mark.parametrize("lq,lk,mask,w", [
    (7, 7, "none", 0), (7, 7, "causal", 0), (3, 10, "causal", 0), (1, 10, "causal", 0),
    (10, 10, "window", 4), (4, 12, "window", 3), (5, 5, "window", 9), (8, 8, "window", 1),
    (64, 200, "window", 100), (300, 300, "window", 1024), (40, 40, "window", 40),
])
def test_visible_pairs_closed_form_matches_oracle_count(lq, lk, mask, w):
    assert bench.visible_pairs(lq, lk, mask, w) == visible_pairs(lq, lk, mask, w)
    s = dict(lq=lq, lk=lk, mask=mask, window=w)
    vm = visible_mask(lq, lk, mask, w)
    for i in range(lq):
        assert bench.row_visible(i, s) == int(vm[i].sum())


def test_workload_table_matches_the_five_workloads():
    names = [s["name"] for s in bench.all_shapes()]
    assert len(names) == 1 + 12 + 20 + 3 + 4 + 5 + 2 + 2 + 3
    assert bench.DEFAULT in names
    s = bench.SHAPES[bench.DEFAULT]
    assert (s["hq"], s["hkv"], s["lq"], s["lk"], s["dqk"], s["dv"], s["dtype"]) == (64, 8, 1, 32768, 192, 128, "bf16")
    assert bench.bound(s) == "hbm"
    assert bench.bound(bench.SHAPES["causal_l32768_d256"]) == "mfma"
    assert bench.bound(bench.SHAPES["verify_lk32768_lq64"]) == "hbm"


def test_window_prefill_flops_and_skip():
    # W=1024 windowed prefill at L=8192, Hq=16, D=256: pairs = W(W+1)/2 + (L-W)W
    s = bench.SHAPES["window_l8192_d256"]
    flops, _ = bench.work(s)
    pairs = 1024 * 1025 // 2 + (8192 - 1024) * 1024
    assert flops == 2 * 16 * 512 * pairs


def test_decode_bytes():
    s = bench.SHAPES["decode_hkv8_lk32768"]
    _, nbytes = bench.work(s)
    assert nbytes == 2 * (64 * 1 * 320 + 8 * 32768 * 320)


def test_multi_gpu_request_exits(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_row_sampler_terminates_when_few_rows_exist():
    from gpu_cases import pick_rows
    assert len(pick_rows(1, 32, 1, 64, 3)) == 32
    assert len(pick_rows(1, 64, 1, 64, 3)) == 64
    rows = pick_rows(1, 16, 8192, 64, 5, window=1024)
    assert len(rows) == 64 and all(0 <= i < 8192 for _, _, i in rows)


def test_mask_array_workloads():
    """The window band handed to the kernel is the oracle's window rule; the
    masked workloads count every pair of their mode and the array's bytes."""
    import numpy as np

    s = bench.SHAPES["maskarr_window_bool_l4096_d256"]
    band = bench.make_mask_array(dict(s, lq=300, lk=500, arr_window=64)).numpy()
    assert (band == visible_mask(300, 500, "window", 64)).all()
    flops, nbytes = bench.work(s)
    assert flops == 2 * 16 * 512 * 4096 * 4096
    assert nbytes == 2 * (16 * 4096 * 512 + 8 * 4096 * 512) + 4096 * 4096
    assert bench.bound(s) == "mfma"
    ref = bench.SHAPES["causal_l4096_d128"]
    s = bench.SHAPES["maskarr_bias_add_causal_l4096_d128"]
    assert bench.work(s)[0] == bench.work(ref)[0]
    assert bench.work(s)[1] == bench.work(ref)[1] + 2 * 4096 * 4096
    s = bench.SHAPES["maskarr_pad_decode_b4_hkv8_lk8192_d128"]
    pad = bench.make_mask_array(s).numpy()
    assert pad.shape == (4, 1, 1, 8192) and pad[..., 0].all()
    lens = pad.sum(axis=-1).ravel()
    assert (pad == (np.arange(8192)[None, None, None, :] < lens[:, None, None, None])).all()
    assert bench.bound(s) == "hbm"
    assert bench.work(s)[1] == bench.work(bench.SHAPES["decode_b4_hkv8_lk8192_d128"])[1] + 4 * 8192


def test_varlen_workload_counts_valid_keys_only():
    s = bench.SHAPES["varlen_decode_b8_hkv8_lk8192_d128"]
    kl = bench.kv_lengths(s)
    assert len(kl) == 8 and all(2048 <= n <= 8192 for n in kl)
    pad = bench.make_mask_array(bench.SHAPES["maskarr_pad_decode_b8_hkv8_lk8192_d128"]).numpy()
    assert pad.sum(axis=-1).ravel().tolist() == kl  # the padding mask keeps the same keys
    _, nbytes = bench.work(s)
    assert nbytes == 2 * (8 * 32 * 256 + 8 * sum(kl) * 256)
    assert bench.bound(s) == "hbm"


def test_vs_baseline_only_for_the_pages_decode_shapes():
    pages = [n for n, s in bench.SHAPES.items() if bench.pages_shape(s)]
    assert sorted(pages) == sorted(f"decode_hkv{h}_lk{lk}" for h in (4, 8)
                                   for lk in (256, 1024, 4096, 8192, 16384, 32768))


def test_backward_workload_counts_five_products():
    s = bench.SHAPES["bwd_causal_l4096_d128"]
    f_fwd, _ = bench.work(bench.SHAPES["causal_l4096_d128"])
    f_bwd, _ = bench.work(s)
    assert f_bwd * 4 == f_fwd * 10  # 2 (3 Dqk + 2 Dv) vs 2 (Dqk + Dv) per pair at Dqk = Dv
    assert bench.bound(s) == "mfma"


@pytest.mark.parametrize("budget", [5.0, 1e-12])
def test_cpu_baseline_reports_the_error_of_the_sampled_rows(budget):
    """The oracle sample of ``cpu_baseline`` doubles as a max-abs error check
    against the runner's output: a stand-in runner whose output is the
    oracle's with one element moved by 0.25 (and one lse by 0.5) must report
    exactly those, on the whole-group path (budget 5 s) and the row-sampled
    path (a budget too small for one group)."""
    import types

    import torch

    from oracle import sdpa_ref
    from scaled_dot_product_fwd_amd.synth import default_scale, make_qkv

    s = bench.shape("tiny", 1, 4, 2, 6, 40, 16, 16, "f32", "causal", 0, 5)
    q, k, v = make_qkv(1, 4, 2, 6, 40, 16, 16, torch.float32, 5)
    scale = default_scale(16)
    ro, rl = sdpa_ref(q, k, v, scale, "causal", 0)
    o = torch.tensor(ro, dtype=torch.float32)
    lse = torch.tensor(rl, dtype=torch.float32)
    o[0, 1, 0, 3] += 0.25  # row 0 is picked by the row sampler too
    lse[0, 2, 0] += 0.5
    run = types.SimpleNamespace(cpu=(q, k, v), scale=scale, o=o, lse=lse, mask_cpu=None)
    out = bench.cpu_baseline(s, run, budget_s=budget)
    err = out["max_abs_err"]
    assert abs(err["o"] - 0.25) < 1e-6 and abs(err["lse"] - 0.5) < 1e-6, err


def test_backward_call_spans_from_a_kernel_trace(tmp_path):
    # two calls whose dQ and dK/dV kernels overlap; a forward kernel between
    # them is not part of either call
    rows = [("void sdpa::dev::bwd_prep_kernel<sdpa::dev::BF16>(sdpa::BwdArgs)", 100, 110),
            ("void sdpa::dev::bwd_dkdv_kernel<sdpa::dev::BF16, 128, false>(sdpa::BwdArgs)", 112, 400),
            ("void sdpa::dev::bwd_dq_kernel<sdpa::dev::BF16, 128, false>(sdpa::BwdArgs)", 111, 350),
            ("void sdpa::dev::attn_fwd_kernel<sdpa::dev::BF16, 128, 128, 4, 1, 64, 2, 0, 1>(sdpa::AttnArgs)", 401, 900),
            ("void sdpa::dev::bwd_prep_kernel<sdpa::dev::BF16>(sdpa::BwdArgs)", 1000, 1010),
            ("void sdpa::dev::bwd_dq_kernel<sdpa::dev::BF16, 128, false>(sdpa::BwdArgs)", 1011, 1500),
            ("void sdpa::dev::bwd_dkdv_kernel<sdpa::dev::BF16, 128, false>(sdpa::BwdArgs)", 1012, 1300)]
    lines = ['"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"']
    lines += [f'"KERNEL_DISPATCH","{n}",{a},{b}' for n, a, b in rows]
    (tmp_path / "run_kernel_trace.csv").write_text("\n".join(lines) + "\n")
    assert bench.bwd_call_spans(str(tmp_path)) == [300, 500]
