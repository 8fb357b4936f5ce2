"""C-ABI boundary on the host (no GPU): exports, validation, planning.

Every validation error is forced from the CPU; none of these calls reaches a
kernel launch (validation runs before any HIP call, and the device check comes
last).  Error messages must name the violated constraint, as the force-fused
contract of mlx PR #4185 "Add force_fused option to
scaled_dot_product_attention" (Validation) asks.
"""

import ctypes
import os
import re

import pytest

import scaled_dot_product_fwd_amd as sdpa
from scaled_dot_product_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sdpa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_desc_init_contiguous_strides():
    d = sdpa.sdpa_desc_init(2, 8, 2, 5, 7, 64, 32, _lib.SDPA_BF16)
    assert list(d.q_stride) == [8 * 5 * 64, 5 * 64, 64]
    assert list(d.k_stride) == [2 * 7 * 64, 7 * 64, 64]
    assert list(d.v_stride) == [2 * 7 * 32, 7 * 32, 32]
    assert list(d.o_stride) == [8 * 5 * 32, 5 * 32, 32]
    assert d.mask == 0 and d.window == 0 and d.num_splits == 0
    assert abs(d.scale - 0.125) < 1e-9


def _desc(b=1, hq=4, hkv=2, lq=8, lk=16, dqk=64, dv=64, dtype=_lib.SDPA_BF16, **kw):
    return sdpa.make_desc((b, hq, lq, dqk), (b, hkv, lk, dqk), (b, hkv, lk, dv), dtype, **kw)


def _status(fn, *args):
    with pytest.raises(sdpa.SdpaError) as ei:
        fn(*args)
    return str(ei.value)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(lq=0), "SDPA_E_SHAPE", "every size must be >= 1"),
    (dict(hq=6, hkv=4), "SDPA_E_SHAPE", "multiple of heads_kv"),
    (dict(dqk=1024, dv=1024), "SDPA_E_HEAD_DIM", "Dqk=1024"),
    (dict(dqk=520, dv=512), "SDPA_E_HEAD_DIM", "from 8 to 512"),
    (dict(dqk=512, dv=512, dtype=_lib.SDPA_F32), "SDPA_E_HEAD_DIM", "float32 supports head dims up to 128"),
    (dict(dqk=512, dv=512, row_tile=128), "SDPA_E_PLAN", "64-row tiles"),
    (dict(dqk=72, dv=76), "SDPA_E_HEAD_DIM", "multiples of 8"),
    (dict(dqk=160, dv=160, dtype=_lib.SDPA_F32), "SDPA_E_HEAD_DIM", "float32 supports head dims up to 128"),
    (dict(dtype=7), "SDPA_E_DTYPE", "dtype"),
    (dict(lq=17, lk=16, mask="causal"), "SDPA_E_MASK", "causal masking requires Lq <= Lk"),
    (dict(lq=17, lk=16, mask="window", window_size=4), "SDPA_E_MASK", "Lq <= Lk"),
    (dict(mask="window", window_size=0), "SDPA_E_MASK", "window >= 1"),
    (dict(mask="causal", window_size=3), "SDPA_E_MASK", "window must be 0"),
    (dict(scale=float("inf")), "SDPA_E_SCALE", "finite"),
    (dict(scale=float("nan")), "SDPA_E_SCALE", "finite"),
    (dict(q_stride=(8 * 8 * 64, 8 * 64, 60)), "SDPA_E_STRIDE", "q_stride[2]"),
    (dict(k_stride=(1 << 30, 1 << 26, (16 << 20) // 2 + 8)), "SDPA_E_STRIDE", "k_stride[2]"),
    (dict(v_stride=(1 << 30, 1 << 26, (16 << 20) // 2 + 8)), "SDPA_E_STRIDE", "v_stride[2]"),
    (dict(num_splits=-1), "SDPA_E_PLAN", "num_splits"),
    (dict(row_tile=48), "SDPA_E_PLAN", "row_tile"),
])
def test_validation_errors_name_the_constraint(kw, code, needle):
    d = _desc(**kw)
    msg = _status(sdpa.sdpa_workspace_bytes, d)
    assert msg.startswith(code), msg
    assert needle in msg, msg
    msg2 = _status(sdpa.sdpa_describe_plan, d)
    assert msg2.startswith(code)
    # forward validates before touching the device: same error, nothing launched
    msg3 = _status(sdpa.sdpa_forward, d, 16, 16, 16, 16, None, None, 0, None)
    assert msg3.startswith(code)


def test_validation_errors_are_value_errors():
    with pytest.raises(ValueError):
        sdpa.sdpa_workspace_bytes(_desc(dqk=1024, dv=1024))


def test_forward_null_pointers():
    msg = _status(sdpa.sdpa_forward, _desc(), 0, 16, 16, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_NULL")


def test_forward_unaligned_pointer():
    msg = _status(sdpa.sdpa_forward, _desc(), 16 + 8, 16, 16, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_STRIDE") and "16-byte aligned" in msg


def test_forward_missing_workspace():
    d = _desc(hq=64, hkv=4, lq=1, lk=32768, dqk=192, dv=128, mask="causal")
    need = sdpa.sdpa_workspace_bytes(d)
    assert need > 0
    msg = _status(sdpa.sdpa_forward, d, 16, 16, 16, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_WORKSPACE") and str(need) in msg
    msg = _status(sdpa.sdpa_forward, d, 16, 16, 16, 16, None, 256, need - 1, None)
    assert msg.startswith("SDPA_E_WORKSPACE")


def test_noalloc_rejects_plans_beyond_its_scratch():
    # 8 KV heads x 64 packed rows x 1024 forced splits x (128 + 2) float32 = 272 MB > 64 MiB:
    # rejected on the host, before any pointer or device is looked at
    d = _desc(hq=64, hkv=8, lq=8, lk=65536, dqk=128, dv=128, num_splits=1024)
    need = sdpa.sdpa_workspace_bytes(d)
    assert need > 64 << 20
    msg = _status(sdpa.sdpa_forward_noalloc, d, 16, 16, 16, None, None, None, 16, None, None)
    assert msg.startswith("SDPA_E_WORKSPACE") and str(need) in msg and str(64 << 20) in msg
    # invalid descriptors fail validation first, as in every other entry point
    msg = _status(sdpa.sdpa_forward_noalloc, _desc(dqk=1024, dv=1024), 16, 16, 16, None, None, None, 16, None,
                  None)
    assert msg.startswith("SDPA_E_HEAD_DIM")


def test_last_error_is_cleared_by_success():
    _status(sdpa.sdpa_workspace_bytes, _desc(dqk=1024, dv=1024))
    assert sdpa.sdpa_last_error() != ""
    sdpa.sdpa_workspace_bytes(_desc())
    assert sdpa.sdpa_last_error() == ""


def _plan(**kw):
    s = sdpa.sdpa_describe_plan(_desc(**kw))
    return dict(tok.split("=", 1) for tok in s.split())


def test_plan_decode_config_splits_keys():
    for hkv in (4, 8):
        for lk in (256, 1024, 4096, 8192, 16384, 32768):
            p = _plan(hq=64, hkv=hkv, lq=1, lk=lk, dqk=192, dv=128, mask="causal")
            assert p["family"] == "decode"
            assert p["mask"] == "none"  # causal with one query sees every key
            assert p["dqk"] == "192->192" and p["dv"] == "128->128"
            splits = int(p["splits"])
            assert splits >= 1 and splits <= (lk + 127) // 128
            if lk >= 8192:
                assert int(p["grid"]) >= 256  # the whole chip streams the keys
            assert (int(p["workspace"]) > 0) == (splits > 1)


@pytest.mark.parametrize("lq,fam,tiles", [(1, "decode", 1), (8, "decode", 1), (12, "short", 1),
                                          (16, "decode", 2), (24, "prefill", 1), (48, "wide", 1),
                                          (64, "wide", 1), (65, "prefill", 3)])
def test_plan_verify_window_family(lq, fam, tiles):
    p = _plan(hq=32, hkv=8, lq=lq, lk=16384, dqk=128, dv=128, dtype=_lib.SDPA_F16)
    assert p["family"] == fam and int(p["row_tiles"]) == tiles
    assert int(p["grid"]) >= 256


def test_plan_small_prefill_grid_takes_64_row_tiles():
    # 16 heads x 8 tiles of 128 rows would leave half of the 256 CUs idle
    p = _plan(hq=16, hkv=16, lq=1024, lk=1024, dqk=72, dv=72)
    assert p["family"] == "short" and p["rows_per_wg"] == "64" and p["grid"] == "256" and p["splits"] == "1"
    # 240 tiles of 128 rows: kept
    p = _plan(hq=20, hkv=20, lq=1500, lk=1500, dqk=64, dv=64)
    assert p["family"] == "prefill" and p["rows_per_wg"] == "128"
    # head dims above 128 and forced tiles: kept
    p = _plan(hq=4, hkv=4, lq=1024, lk=1024, dqk=256, dv=256)
    assert p["family"] == "prefill" and p["rows_per_wg"] == "128"
    p = _plan(hq=16, hkv=16, lq=1024, lk=1024, dqk=72, dv=72, row_tile=128)
    assert p["rows_per_wg"] == "128"


def test_plan_prefill_configs_do_not_split():
    p = _plan(hq=20, hkv=20, lq=1500, lk=1500, dqk=64, dv=64)
    assert p["family"] == "prefill" and p["splits"] == "1" and p["workspace"] == "0"
    p = _plan(hq=16, hkv=16, lq=4096, lk=4096, dqk=72, dv=72)
    assert p["dqk"] == "72->80" and p["dv"] == "72->96"
    p = _plan(hq=16, hkv=2, lq=32768, lk=32768, dqk=256, dv=256, mask="causal")
    assert p["splits"] == "1" and p["mask"] == "causal"


def test_plan_head_dim_padding():
    # QK pads to the 16-deep MFMA step where an (80, 96) kernel exists; PV to
    # whole 32-wide tiles; float32 keeps 32-wide padding on both.
    for dqk, dv, want in ((72, 72, ("80", "96")), (80, 80, ("80", "96")), (80, 96, ("80", "96")),
                          (72, 64, ("80", "96")), (64, 96, ("80", "96")), (88, 88, ("96", "96")),
                          (64, 64, ("64", "64")), (40, 40, ("64", "64"))):
        for lq in (1, 16, 200, 4096):
            p = _plan(hq=16, hkv=4, lq=lq, lk=4096, dqk=dqk, dv=dv)
            assert (p["dqk"], p["dv"]) == (f"{dqk}->{want[0]}", f"{dv}->{want[1]}"), (dqk, dv, lq, p)
    p = _plan(hq=16, hkv=4, lq=200, lk=4096, dqk=72, dv=72, dtype=_lib.SDPA_F32)
    assert (p["dqk"], p["dv"]) == ("72->96", "72->96")


def test_plan_canonical_masks():
    assert _plan(lq=8, lk=16, mask="window", window_size=16)["mask"] == "causal"
    assert _plan(lq=8, lk=16, mask="window", window_size=100)["mask"] == "causal"
    assert _plan(lq=8, lk=16, mask="window", window_size=15)["mask"] == "window(15)"
    assert _plan(lq=1, lk=16, mask="causal")["mask"] == "none"


def test_plan_overrides():
    p = _plan(hq=32, hkv=8, lq=4, lk=4096, num_splits=3, row_tile=128)
    assert p["splits"] == "3" and p["rows_per_wg"] == "128" and p["family"] == "prefill"
    p = _plan(hq=32, hkv=8, lq=4, lk=4096, num_splits=1)
    assert p["splits"] == "1" and p["workspace"] == "0"


def test_forward_without_gpu_tensors_raises():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError, match="there is no CPU path"):
        sdpa.forward(q, q, q)


def test_split_workspace_layout():
    # per packed row and split: the unnormalised partial output in float32,
    # then an (m, l) float32 pair
    rows = 2 * 16 * 1
    for dtype in (_lib.SDPA_BF16, _lib.SDPA_F16, _lib.SDPA_F32):
        d = _desc(b=2, hq=16, hkv=4, lq=1, lk=5000, dqk=64, dv=64, num_splits=16, dtype=dtype)
        o_bytes = (rows * 16 * 64 * 4 + 255) // 256 * 256
        assert sdpa.sdpa_workspace_bytes(d) == o_bytes + rows * 16 * 8


def test_plan_xcd_grouping():
    p = _plan(hq=32, hkv=8, lq=96, lk=32768, dqk=128, dv=128, dtype=_lib.SDPA_F16)
    assert int(p["row_tiles"]) == 3 and int(p["splits"]) > 1 and p["xcd_group"] == "8"
    # one row tile per KV head, 8 KV heads: each head's splits on one XCD,
    # the combine's rows of that head on the same XCD
    p = _plan(hq=64, hkv=8, lq=1, lk=32768, dqk=192, dv=128)
    assert p["xcd_group"] == p["splits"] and int(p["splits"]) > 1 and p["combine_xcd"] == "1"
    p = _plan(hq=32, hkv=4, lq=1, lk=32768, dqk=128, dv=128)
    assert int(p["splits"]) > 1 and p["xcd_group"] == "0" and p["combine_xcd"] == "0"
    p = _plan(hq=16, hkv=8, lq=4096, lk=4096, dqk=256, dv=256, mask="window", window_size=1024)
    assert p["splits"] == "1" and p["xcd_group"] == "0"  # two rounds of tiles only
    p = _plan(hq=16, hkv=8, lq=8192, lk=8192, dqk=256, dv=256, mask="window", window_size=1024)
    assert p["splits"] == "1" and p["xcd_group"] == "8"
    p = _plan(hq=16, hkv=2, lq=32768, lk=32768, dqk=256, dv=256, mask="causal")
    assert p["xcd_group"] == "0"
    # unmasked prefill: the row tiles of one head in one group (the largest
    # divisor of the tiles per head that tiles the grid in groups of 8)
    p = _plan(hq=16, hkv=16, lq=4096, lk=4096, dqk=72, dv=72)
    assert p["row_tiles"] == "32" and p["grid"] == "512" and p["xcd_group"] == "32"
    p = _plan(hq=20, hkv=20, lq=1500, lk=1500, dqk=64, dv=64)
    assert p["row_tiles"] == "12" and p["grid"] == "240" and p["xcd_group"] == "6"
    p = _plan(hq=13, hkv=13, lq=1500, lk=1500, dqk=64, dv=64)  # 156 tiles: no group of 8 fits
    assert p["splits"] == "1" and p["xcd_group"] == "0"


def test_split_rows_beyond_one_grid_fall_back_to_unsplit():
    # B*Hq*Lq = 2^31 rows would need more combine workgroups than a grid holds
    kw = dict(b=4, hq=256, hkv=1, lq=1 << 21, lk=1 << 21, dqk=64, dv=64)
    p = _plan(**kw)
    assert p["splits"] == "1"
    msg = _status(sdpa.sdpa_workspace_bytes, _desc(num_splits=2, **kw))
    assert "SDPA_E_PLAN" in msg and "2^31" in msg


# ---------------------------------------------------------------------------
# Explicit mask arrays
# ---------------------------------------------------------------------------

def test_desc_struct_layout_matches_the_header(tmp_path):
    """ctypes mirror of sdpa_desc_t: every field offset and the size agree with
    what the C compiler makes of include/sdpa.h."""
    fields = [f for f, _ in _lib.sdpa_desc_t._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "sdpa.h"\nint main(void){\n' +
                   "".join(f'printf("%zu\\n", offsetof(sdpa_desc_t, {f}));\n' for f in fields) +
                   'printf("%zu\\n", sizeof(sdpa_desc_t));\nreturn 0;}\n')
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    want = [getattr(_lib.sdpa_desc_t, f).offset for f in fields] + [ctypes.sizeof(_lib.sdpa_desc_t)]
    assert got == want


@pytest.mark.parametrize("kw,code,needle", [
    (dict(mask_array=3), "SDPA_E_MASK", "mask_array must be"),
    (dict(mask_array=_lib.SDPA_MASK_ARRAY_BOOL, mask_stride=(0, 0, 8)), "SDPA_E_STRIDE", "mask_stride[2]"),
    (dict(mask_array=_lib.SDPA_MASK_ARRAY_ADD, mask_stride=(0, 4, 16)), "SDPA_E_STRIDE", "mask_stride[1]"),
    (dict(mask_array=_lib.SDPA_MASK_ARRAY_BOOL, mask_stride=(-16, 0, 16)), "SDPA_E_STRIDE", "mask_stride[0]"),
])
def test_mask_array_validation(kw, code, needle):
    d = _desc(**kw)
    msg = _status(sdpa.sdpa_workspace_bytes, d)
    assert msg.startswith(code) and needle in msg, msg
    msg = _status(sdpa.sdpa_forward_masked, d, 16, 16, 16, 16, 16, None, None, 0, None)
    assert msg.startswith(code), msg


def test_mask_array_pointer_must_match_the_desc():
    d = _desc(mask_array=_lib.SDPA_MASK_ARRAY_BOOL, mask_stride=(0, 0, 16))
    msg = _status(sdpa.sdpa_forward_masked, d, 16, 16, 16, None, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_NULL") and "mask is NULL" in msg
    msg = _status(sdpa.sdpa_forward_masked, _desc(), 16, 16, 16, 16, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_NULL") and "SDPA_MASK_ARRAY_NONE" in msg
    msg = _status(sdpa.sdpa_forward_masked, d, 16, 16, 16, 24, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_STRIDE") and "16-byte aligned" in msg
    # the plain entry point refuses a desc that names an array
    msg = _status(sdpa.sdpa_forward, d, 16, 16, 16, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_MASK") and "sdpa_forward_masked" in msg


@pytest.mark.parametrize("dtype,d,kind,family,bk", [
    # prefill: the mask tile joins K and V in LDS; 64-key blocks while two
    # workgroups still fit a CU, else 32-key blocks (large dims keep 64 with
    # an array; without one, both head dims from 192 take 32-key blocks for
    # the pipelined loop)
    (_lib.SDPA_BF16, 128, _lib.SDPA_MASK_ARRAY_NONE, "prefill", "64"),
    (_lib.SDPA_BF16, 128, _lib.SDPA_MASK_ARRAY_BOOL, "prefill", "64"),
    (_lib.SDPA_BF16, 128, _lib.SDPA_MASK_ARRAY_ADD, "prefill", "32"),
    (_lib.SDPA_BF16, 256, _lib.SDPA_MASK_ARRAY_ADD, "prefill", "64"),
    (_lib.SDPA_BF16, 256, _lib.SDPA_MASK_ARRAY_NONE, "prefill", "32"),
    (_lib.SDPA_F32, 128, _lib.SDPA_MASK_ARRAY_ADD, "prefill", "32"),
])
def test_plan_masked_prefill_family(dtype, d, kind, family, bk):
    # (16 heads: enough 128-row tiles that no shape here moves to 64-row tiles)
    p = _plan(b=1, hq=16, hkv=16, lq=2048, lk=2048, dqk=d, dv=d, dtype=dtype, mask_array=kind,
              mask_stride=(0, 0, 2048))
    assert p["family"] == family and p["block_keys"] == bk
    if kind != _lib.SDPA_MASK_ARRAY_NONE:
        assert p["mask_array"] == ("bool" if kind == _lib.SDPA_MASK_ARRAY_BOOL else "add")
    assert int(p["lds"]) <= 160 * 1024


def test_plan_masked_decode_keeps_lds_within_a_cu():
    for d in (64, 128, 160, 256):
        for kind in (_lib.SDPA_MASK_ARRAY_BOOL, _lib.SDPA_MASK_ARRAY_ADD):
            p = _plan(b=1, hq=32, hkv=8, lq=1, lk=8192, dqk=d, dv=d, mask_array=kind,
                      mask_stride=(0, 0, 0))
            assert p["family"] == "decode" and int(p["lds"]) <= 160 * 1024
    # D=160 decode: 4x32-key waves fit without a mask array, not with an additive one
    assert _plan(hq=32, hkv=8, lq=1, lk=8192, dqk=160, dv=160)["block_keys"] == "128"
    assert _plan(hq=32, hkv=8, lq=1, lk=8192, dqk=160, dv=160, mask_array=_lib.SDPA_MASK_ARRAY_ADD,
                 mask_stride=(0, 0, 0))["block_keys"] == "64"


def test_mask_layout_host_checks():
    import torch

    q = torch.zeros(2, 4, 5, 8, dtype=torch.bfloat16)
    good = sdpa.pad_mask(torch.ones(5, 13, dtype=torch.bool))
    assert good.shape == (5, 13) and good.stride() == (16, 1)
    kind, st = sdpa._mask_layout(good, q, 2, 4, 5, 13)
    assert kind == _lib.SDPA_MASK_ARRAY_BOOL and st == [0, 0, 16]
    add = sdpa.pad_mask(torch.zeros(2, 1, 5, 13), dtype=torch.bfloat16)
    kind, st = sdpa._mask_layout(add, q, 2, 4, 5, 13)
    assert kind == _lib.SDPA_MASK_ARRAY_ADD and st == [5 * 16, 0, 16]
    with pytest.raises(sdpa.SdpaValueError, match="16-byte"):
        sdpa._mask_layout(torch.ones(5, 13, dtype=torch.bool), q, 2, 4, 5, 13)
    with pytest.raises(sdpa.SdpaValueError, match="readable"):
        # rows start on 16-byte boundaries, but the storage ends 3 bytes
        # short of the last row's 16-byte rounding
        sdpa._mask_layout(torch.ones(77, dtype=torch.bool).as_strided((5, 13), (16, 1)), q, 2, 4, 5, 13)
    with pytest.raises(sdpa.SdpaValueError, match="broadcast"):
        sdpa._mask_layout(good[:4], q, 2, 4, 5, 13)
    with pytest.raises(sdpa.SdpaValueError, match="dtype"):
        sdpa._mask_layout(torch.zeros(5, 16, dtype=torch.float32), q, 2, 4, 5, 16)


def test_varlen_length_arrays_must_be_aligned():
    d = _desc()
    msg = _status(sdpa.sdpa_forward_varlen, d, 16, 16, 16, None, 18, None, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_STRIDE") and "q_lens" in msg
    msg = _status(sdpa.sdpa_forward_varlen, d, 16, 16, 16, None, None, 22, 16, None, None, 0, None)
    assert msg.startswith("SDPA_E_STRIDE") and "kv_lens" in msg


@pytest.mark.parametrize("lq,dqk,dv", [(1, 512, 512), (8, 512, 512), (4096, 512, 512), (300, 320, 320),
                                       (16, 512, 256)])
def test_plan_head_dim_512(lq, dqk, dv):
    """Head dims above 256 run the 512 instance: two 32-row groups whose waves
    split the dv tiles, 32-key blocks (two buffers of 64 KB), any query length."""
    p = _plan(b=1, hq=32, hkv=8, lq=lq, lk=8192, dqk=dqk, dv=dv, mask="causal")
    assert p["family"] == "prefill" and p["rows_per_wg"] == "64" and p["waves"] == "2x1x2"
    assert p["block_keys"] == "32" and p["dqk"].endswith("->512") and p["dv"].endswith("->512")
    assert int(p["lds"]) == 2 * 32 * 2048 + 4 * 4096  # + the pairs' partial-score exchange
    if lq == 1:
        assert int(p["splits"]) > 1  # a decode call still spreads its keys over the chip


@pytest.mark.parametrize("b,hq,hkv,lq", [(1, 4, 2, 200), (1, 4, 2, 1), (2, 8, 2, 130), (1, 2, 1, 257)])
def test_backward_workspace_covers_whole_row_blocks(b, hq, hkv, lq):
    """Per (batch, KV head) the workspace holds lse2 and D for Rp packed rows,
    Rp = G * Lq rounded up to the dK/dV kernel's 32-row block, then Rp query
    indices: a block's tile of them never leaves its entry.  (One row part:
    more add their float32 partials after this, see the row-part test.)"""
    d = _desc(b=b, hq=hq, hkv=hkv, lq=lq, lk=300, dqk=64, dv=64, mask="causal", num_splits=1)
    rp = -(-(hq // hkv) * lq // 32) * 32
    want = -(-(2 * b * hkv * rp + rp) * 4 // 256) * 256
    assert sdpa.sdpa_backward_workspace_bytes(d) == want


def test_backward_validation():
    for kw, code, needle in [(dict(dtype=_lib.SDPA_F32), "SDPA_E_DTYPE", "float16 and bfloat16"),
                             (dict(dqk=256, dv=256), "SDPA_E_HEAD_DIM", "up to 128")]:
        msg = _status(sdpa.sdpa_backward_workspace_bytes, _desc(**kw))
        assert msg.startswith(code) and needle in msg, msg
    # a mask array is planned like the forward's (its strides are checked there)
    d = _desc(mask_array=_lib.SDPA_MASK_ARRAY_BOOL, mask_stride=(0, 0, 16))
    assert sdpa.sdpa_backward_workspace_bytes(d) > 0


def test_plan_wide_family_limits():
    # 128 < R <= 256 with head dims up to 128: one 256-row tile
    p = _plan(hq=8, hkv=1, lq=30, lk=4096, dqk=128, dv=128)
    assert p["family"] == "wide" and p["rows_per_wg"] == "256" and p["waves"] == "8x1"
    # larger dims keep 128-row tiles; forcing 256 there is refused
    assert _plan(hq=8, hkv=1, lq=30, lk=4096, dqk=256, dv=256)["family"] == "prefill"
    msg = _status(sdpa.sdpa_workspace_bytes, _desc(hq=8, hkv=1, lq=30, lk=4096, dqk=256, dv=256, row_tile=256))
    assert msg.startswith("SDPA_E_PLAN") and "row_tile 256" in msg
    assert _plan(hq=8, hkv=1, lq=30, lk=4096, dqk=128, dv=128, dtype=_lib.SDPA_F32)["family"] == "prefill"
    assert _plan(hq=8, hkv=1, lq=30, lk=4096, dqk=96, dv=96, dtype=_lib.SDPA_F32)["family"] == "wide"
    # an additive mask array keeps the LDS within one workgroup's 160 KB
    p = _plan(hq=8, hkv=1, lq=30, lk=4096, dqk=96, dv=96, dtype=_lib.SDPA_F32,
              mask_array=_lib.SDPA_MASK_ARRAY_ADD, mask_stride=(0, 0, 4096))
    assert p["family"] == "wide" and int(p["lds"]) <= 160 * 1024


def test_backward_varlen_validates_before_any_launch():
    """The per-length / masked backward shares the backward's checks, in
    order, and returns before touching the device: missing pointers, the
    plan, the mask pointer against the descriptor, alignment, workspace."""
    d = _desc(b=2, hq=4, hkv=2, lq=8, lk=16, dqk=64, dv=64, mask="causal")
    ptr = 1 << 20  # aligned, never dereferenced on the host
    bwd = sdpa.sdpa_backward_varlen

    def call(desc, q=ptr, mask=0, ws_bytes=1 << 20):
        return _status(bwd, desc, q, ptr, ptr, mask, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ws_bytes, 0)

    assert call(d, q=0).startswith("SDPA_E_NULL")
    assert call(_desc(dtype=_lib.SDPA_F32)).startswith("SDPA_E_DTYPE")
    assert call(d, mask=ptr).startswith("SDPA_E_NULL")  # a mask the descriptor does not name
    dm = _desc(b=2, hq=4, hkv=2, lq=8, lk=16, dqk=64, dv=64, mask_array=_lib.SDPA_MASK_ARRAY_BOOL,
               mask_stride=(0, 0, 16))
    assert call(dm).startswith("SDPA_E_NULL")  # the descriptor names a mask that is missing
    assert call(d, q=ptr + 8).startswith("SDPA_E_STRIDE")
    assert call(d, ws_bytes=16).startswith("SDPA_E_WORKSPACE")
    # the plain backward refuses a descriptor with a mask array
    msg = _status(sdpa.sdpa_backward, dm, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, 1 << 20, 0)
    assert msg.startswith("SDPA_E_MASK"), msg


def _bwd_ws(hq, hkv, l, d, mask, parts=0):
    desc = _desc(hq=hq, hkv=hkv, lq=l, lk=l, dqk=d, dv=d, mask=mask, num_splits=parts)
    return sdpa.sdpa_backward_workspace_bytes(desc)


def test_bwd_plan_row_parts():
    """The dK/dV row parts show in the workspace: [lse2][D][query index]
    rounded to 256 bytes, then parts x B*Hkv x Lk x (Dqk + Dv) float32."""
    def base(hq, hkv, l):
        z, rp = hkv, -(-(hq // hkv) * l // 32) * 32
        return ((2 * z * rp + rp) * 4 + 255) // 256 * 256

    # MHA causal L=4096 (512 key tiles, balanced by heaviest-first): no parts
    assert _bwd_ws(16, 16, 4096, 128, "causal") == base(16, 16, 4096)
    # GQA causal L=4096, Hkv=8 (256 tiles, the first 32x longer than the last): 2 parts
    assert _bwd_ws(32, 8, 4096, 128, "causal") == base(32, 8, 4096) + 2 * 8 * 4096 * 256 * 4
    # forced counts, and the limit
    assert _bwd_ws(32, 8, 4096, 128, "causal", parts=1) == base(32, 8, 4096)
    assert _bwd_ws(4, 2, 300, 64, "none", parts=5) == base(4, 2, 300) + 5 * 2 * 300 * 128 * 4
    with pytest.raises(sdpa.SdpaError, match="row parts"):
        _bwd_ws(4, 2, 300, 64, "none", parts=65)
    # small shapes keep at least 8 row blocks per part: a 16-row tile gets none
    assert _bwd_ws(4, 2, 16, 64, "causal") == base(4, 2, 16)
