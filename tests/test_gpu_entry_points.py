"""The plain C entry points launched for real through ctypes.

``forward()`` goes through ``sdpa_forward_varlen``; these tests call
``sdpa_forward`` (mlx PR #4185, API: the fused forward) and
``sdpa_forward_masked`` (mlx PR #3552, Public API: the mask array beside the
mask mode) themselves, with caller-owned outputs and workspace, and hold the
results to the oracle's tolerances on every element.
"""

import numpy as np
import pytest
import torch

import scaled_dot_product_fwd_amd as sdpa
from gpu_cases import TOL_LSE, TOL_O, lse_err
from oracle import sdpa_ref
from scaled_dot_product_fwd_amd.synth import DTYPES, additive_mask, bool_mask, default_scale, make_qkv

pytestmark = pytest.mark.gpu


def _buffers(q, k, v, desc):
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    b, hq, lq, _ = q.shape
    o = torch.full((b, hq, lq, v.shape[3]), float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full((b, hq, lq), float("nan"), dtype=torch.float32, device=dev)
    ws_bytes = sdpa.sdpa_workspace_bytes(desc)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    return qd, kd, vd, o, lse, ws, ws_bytes


def _check(o, lse, ro, rl, dt):
    go = o.cpu().to(torch.float64).numpy()
    gl = lse.cpu().to(torch.float64).numpy()
    assert not np.isnan(go).any() and not np.isnan(gl).any(), "unwritten output"
    assert float(np.abs(go - ro).max()) <= TOL_O[dt]
    assert lse_err(gl, rl) <= TOL_LSE[dt]


@pytest.mark.parametrize("case", [
    # (B, Hq, Hkv, Lq, Lk, D, dtype, mask, window): an unsplit prefill and a split decode
    (2, 8, 2, 100, 300, 64, "bf16", "causal", 0),
    (1, 16, 4, 1, 4096, 128, "f16", "none", 0),
    (1, 4, 4, 70, 500, 32, "f32", "window", 50),
])
def test_sdpa_forward_entry_point(case):
    b, hq, hkv, lq, lk, d, dtype, mask, window = case
    print("CASE sdpa_forward", case, flush=True)
    dt = DTYPES[dtype]
    q, k, v = make_qkv(b, hq, hkv, lq, lk, d, d, dt, 9300 + lq)
    scale = default_scale(d)
    desc = sdpa.make_desc(q.shape, k.shape, v.shape, sdpa._dtype_code(dt), scale=scale, mask=mask,
                          window_size=window)
    qd, kd, vd, o, lse, ws, ws_bytes = _buffers(q, k, v, desc)
    stream = torch.cuda.current_stream().cuda_stream
    sdpa.sdpa_forward(desc, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      ws.data_ptr() if ws_bytes else None, ws_bytes, stream)
    torch.cuda.synchronize()
    ro, rl = sdpa_ref(q, k, v, scale, mask, window)
    _check(o, lse, ro, rl, dt)


@pytest.mark.parametrize("kind", ["bool", "add"])
def test_sdpa_forward_masked_entry_point(kind):
    b, hq, hkv, lq, lk, d = 1, 8, 2, 64, 257, 64
    print("CASE sdpa_forward_masked", kind, flush=True)
    dt = torch.bfloat16
    q, k, v = make_qkv(b, hq, hkv, lq, lk, d, d, dt, 9400)
    if kind == "bool":
        arr = bool_mask((lq, lk), 9401, 0.7)
        code = sdpa.SDPA_MASK_ARRAY_BOOL
    else:
        arr = additive_mask((lq, lk), 9402, dt)
        code = sdpa.SDPA_MASK_ARRAY_ADD
    scale = default_scale(d)
    dev = torch.device("cuda", 0)
    md = sdpa.pad_mask(arr.to(dev))
    desc = sdpa.make_desc(q.shape, k.shape, v.shape, sdpa._dtype_code(dt), scale=scale, mask="causal",
                          mask_array=code, mask_stride=(0, 0, md.stride(0)))
    qd, kd, vd, o, lse, ws, ws_bytes = _buffers(q, k, v, desc)
    stream = torch.cuda.current_stream().cuda_stream
    sdpa.sdpa_forward_masked(desc, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), md.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), ws.data_ptr() if ws_bytes else None, ws_bytes, stream)
    torch.cuda.synchronize()
    ro, rl = sdpa_ref(q, k, v, scale, "causal", 0, mask_arr=arr)
    _check(o, lse, ro, rl, dt)
