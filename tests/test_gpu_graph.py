"""The forward, split plans with their combine included, can be captured in a
HIP graph (torch.cuda.CUDAGraph on ROCm) and replayed: the library allocates
nothing, clears nothing with a memset, and launches every kernel on the
caller's stream.  Each replay, with new inputs copied into the captured
buffers and eager work between replays, must equal the eager call bitwise
(a fixed plan is deterministic)."""

import numpy as np
import pytest
import torch

import scaled_dot_product_fwd_amd as sdpa
from scaled_dot_product_fwd_amd.synth import default_scale, make_qkv

pytestmark = pytest.mark.gpu


def _say(*a):
    print("CASE", *a, flush=True)


@pytest.mark.parametrize("shape", [
    # b, hq, hkv, lq, lk, d, mask: a split decode (attention + combine) and an unsplit prefill
    (1, 64, 8, 1, 8192, 128, "causal"),
    (1, 8, 2, 300, 300, 64, "causal"),
])
def test_forward_replays_in_a_graph(shape):
    b, hq, hkv, lq, lk, d, mask = shape
    _say("graph", shape)
    dev = torch.device("cuda", 0)
    scale = default_scale(d)
    q, k, v = (t.to(dev) for t in make_qkv(b, hq, hkv, lq, lk, d, d, torch.bfloat16, 21))
    out = torch.empty((b, hq, lq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((b, hq, lq), dtype=torch.float32, device=dev)
    desc = sdpa.make_desc(q.shape, k.shape, v.shape, sdpa.SDPA_BF16, scale=scale, mask=mask)
    ws = torch.empty(max(sdpa.sdpa_workspace_bytes(desc), 256), dtype=torch.uint8, device=dev)
    kw = dict(scale=scale, mask=mask, return_lse=True, out=out, lse_out=lse, workspace=ws)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        sdpa.forward(q, k, v, **kw)  # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sdpa.forward(q, k, v, **kw)

    for rep in range(3):
        q2, k2, v2 = make_qkv(b, hq, hkv, lq, lk, d, d, torch.bfloat16, 100 + rep)
        q.copy_(q2.to(dev))
        k.copy_(k2.to(dev))
        v.copy_(v2.to(dev))
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = out.clone(), lse.clone()
        ref_o, ref_l = sdpa.forward(q, k, v, scale=scale, mask=mask, return_lse=True)  # eager, in between
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o), f"replay {rep}: o differs from the eager call"
        assert torch.equal(got_l, ref_l), f"replay {rep}: lse differs from the eager call"
        assert not np.isnan(got_o.float().cpu().numpy()).any()


@pytest.mark.parametrize("shape", [
    # b, hq, hkv, l, d, mask: one dK/dV part per key tile, and grouped queries with row parts
    (1, 8, 8, 384, 64, "causal"),
    (1, 16, 2, 512, 128, "causal"),
])
def test_backward_replays_in_a_graph(shape):
    """The backward call runs dQ on the library's second stream (forked after
    the prep kernel, joined before the call returns); captured in a graph the
    fork and join become graph edges, and every replay equals the eager call
    bitwise (the backward is deterministic)."""
    b, hq, hkv, l, d, mask = shape
    _say("graph backward", shape)
    dev = torch.device("cuda", 0)
    scale = default_scale(d)
    q, k, v = (t.to(dev) for t in make_qkv(b, hq, hkv, l, l, d, d, torch.bfloat16, 31))
    dout = torch.randn((b, hq, l, d), generator=torch.Generator().manual_seed(32)).to(torch.bfloat16).to(dev)
    o, lse = sdpa.forward(q, k, v, scale=scale, mask=mask, return_lse=True)
    desc = sdpa.make_desc(q.shape, k.shape, v.shape, sdpa.SDPA_BF16, scale=scale, mask=mask)
    ws = torch.empty(sdpa.sdpa_backward_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    grads = [torch.empty_like(t) for t in (q, k, v)]
    kw = dict(scale=scale, mask=mask, dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        sdpa.backward(q, k, v, o, dout, lse, **kw)  # warm-up on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sdpa.backward(q, k, v, o, dout, lse, **kw)

    for rep in range(3):
        q2, k2, v2 = make_qkv(b, hq, hkv, l, l, d, d, torch.bfloat16, 200 + rep)
        q.copy_(q2.to(dev))
        k.copy_(k2.to(dev))
        v.copy_(v2.to(dev))
        o2, lse2 = sdpa.forward(q, k, v, scale=scale, mask=mask, return_lse=True)
        o.copy_(o2)
        lse.copy_(lse2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in grads]
        ref = sdpa.backward(q, k, v, o, dout, lse, scale=scale, mask=mask)  # eager, in between
        torch.cuda.synchronize()
        for name, x, y in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(x, y), f"replay {rep}: {name} differs from the eager call"
            assert not torch.isnan(x.float()).any()
