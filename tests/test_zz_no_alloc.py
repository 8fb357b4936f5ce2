"""The forward that allocates nothing (``sdpa_forward_noalloc``) against the
workspace forward (``sdpa_forward_varlen``) through the C ABI.

Both run the same plan and kernels, so their outputs must agree bit for bit;
each is also held to the oracle's tolerances.  Two calls in a row, the second
on a smaller input, check that the shared per-device scratch carries nothing
from one call into the next.
"""

import numpy as np
import pytest
import torch

import scaled_dot_product_fwd_amd as sdpa
from gpu_cases import TOL_LSE, TOL_O, lse_err
from oracle import sdpa_ref, sdpa_ref_varlen
from scaled_dot_product_fwd_amd.synth import DTYPES, default_scale, make_qkv

pytestmark = pytest.mark.gpu


def _run_both(b, hq, hkv, lq, lk, d, dtype, mask, seed, kv_lens=None, num_splits=0):
    print("CASE noalloc", b, hq, hkv, lq, lk, d, dtype, mask, kv_lens, num_splits, flush=True)
    dt = DTYPES[dtype]
    dev = torch.device("cuda", 0)
    q, k, v = make_qkv(b, hq, hkv, lq, lk, d, d, dt, seed)
    scale = default_scale(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    desc = sdpa.make_desc(qd.shape, kd.shape, vd.shape, sdpa._dtype_code(dt), scale=scale, mask=mask,
                          num_splits=num_splits)
    plan = sdpa.sdpa_describe_plan(desc)
    ws_bytes = sdpa.sdpa_workspace_bytes(desc)
    kvl = None if kv_lens is None else torch.tensor(kv_lens, dtype=torch.int32, device=dev)
    kvp = None if kvl is None else kvl.data_ptr()
    stream = torch.cuda.current_stream(dev).cuda_stream
    outs = []
    for noalloc in (False, True):
        o = torch.full((b, hq, lq, d), float("nan"), dtype=dt, device=dev)
        lse = torch.full((b, hq, lq), float("nan"), dtype=torch.float32, device=dev)
        if noalloc:
            sdpa.sdpa_forward_noalloc(desc, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), None, None, kvp,
                                      o.data_ptr(), lse.data_ptr(), stream)
        else:
            ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
            sdpa.sdpa_forward_varlen(desc, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), None, None, kvp,
                                     o.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws_bytes, stream)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    (o_ws, l_ws), (o_na, l_na) = outs
    assert torch.equal(o_ws.view(torch.int16 if dt != torch.float32 else torch.int32),
                       o_na.view(torch.int16 if dt != torch.float32 else torch.int32)), plan
    assert torch.equal(l_ws.view(torch.int32), l_na.view(torch.int32)), plan
    if kv_lens is None:
        ro, rl = sdpa_ref(q, k, v, scale, mask, 0)
    else:
        ro, rl = sdpa_ref_varlen(q, k, v, scale, mask, 0, kv_lens=kv_lens)
    go = o_na.to(torch.float64).numpy()
    gl = l_na.to(torch.float64).numpy()
    assert not np.isnan(go).any() and not np.isnan(gl).any()
    assert float(np.abs(go - ro).max()) <= TOL_O[dt]
    assert lse_err(gl, rl) <= TOL_LSE[dt]
    return plan, ws_bytes


def test_noalloc_matches_workspace_forward_two_calls():
    # a split decode plan, then a smaller split plan reusing the same scratch
    plan1, ws1 = _run_both(1, 16, 4, 1, 8192, 128, "bf16", "causal", seed=9100)
    assert "splits=1 " not in plan1 and ws1 > 0
    plan2, ws2 = _run_both(1, 8, 2, 3, 1000, 64, "f16", "none", seed=9101, num_splits=5)
    assert "splits=5" in plan2 and 0 < ws2 < ws1


def test_noalloc_per_batch_lengths_and_unsplit():
    _run_both(3, 8, 4, 1, 4096, 128, "bf16", "none", seed=9102, kv_lens=[4096, 17, 2500])
    plan, ws = _run_both(1, 16, 16, 1024, 1024, 64, "bf16", "causal", seed=9103)
    assert ws == 0, plan
