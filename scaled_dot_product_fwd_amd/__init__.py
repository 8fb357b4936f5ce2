"""MI355X (gfx950) fused scaled-dot-product attention forward.

``forward(q, k, v, ...)`` computes ``softmax(scale * q k^T + mask) v`` with the
HIP kernels of ``libsdpa_fwd.so`` (see ``include/sdpa.h``).  PyTorch supplies
device memory and the current stream only; there is no CPU or PyTorch
fallback, and a missing library raises.

Python mirrors the Python API described in mlx PR #4185 "Add force_fused
option to scaled_dot_product_attention" (API) and the ``window_size`` keyword
of mlx PR #3552 "feat(fast): add sliding-window SDPA kernel path" (Public
API).
"""

from __future__ import annotations

import math
from typing import Optional, Tuple, Union

from ._lib import (SDPA_BF16, SDPA_F16, SDPA_F32, SDPA_MASK_ARRAY_ADD,  # noqa: F401
                   SDPA_MASK_ARRAY_BOOL, SDPA_MASK_ARRAY_NONE, SDPA_MASK_CAUSAL, SDPA_MASK_NONE,
                   SDPA_MASK_WINDOW, SdpaError, SdpaRuntimeError, SdpaValueError, load,
                   sdpa_desc_init, sdpa_desc_t, sdpa_describe_plan, sdpa_forward,
                   sdpa_backward, sdpa_backward_varlen, sdpa_backward_workspace_bytes, sdpa_forward_masked,
                   sdpa_forward_noalloc, sdpa_forward_varlen, sdpa_last_error, sdpa_set_profile_events,
                   sdpa_workspace_bytes)

__all__ = ["forward", "backward", "sdpa_backward", "sdpa_backward_varlen", "sdpa_backward_workspace_bytes", "make_desc", "plan_for", "workspace_for", "pad_mask", "sdpa_forward",
           "sdpa_forward_masked", "sdpa_forward_varlen", "sdpa_forward_noalloc", "sdpa_workspace_bytes", "sdpa_describe_plan", "sdpa_last_error",
           "sdpa_desc_init", "sdpa_set_profile_events",
           "SdpaError", "SdpaValueError", "SdpaRuntimeError"]

_MASKS = {"none": SDPA_MASK_NONE, "causal": SDPA_MASK_CAUSAL, "window": SDPA_MASK_WINDOW}


def _dtype_code(dtype) -> int:
    import torch

    codes = {torch.float32: SDPA_F32, torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16}
    if dtype not in codes:
        raise SdpaValueError(f"SDPA_E_DTYPE: unsupported dtype {dtype}")
    return codes[dtype]


def make_desc(q_shape, k_shape, v_shape, dtype: int, *, scale: Optional[float] = None,
              mask: str = "none", window_size: int = 0, q_stride=None, k_stride=None,
              v_stride=None, o_stride=None, num_splits: int = 0, row_tile: int = 0,
              mask_array: int = SDPA_MASK_ARRAY_NONE, mask_stride=(0, 0, 0)) -> sdpa_desc_t:
    """Build a descriptor from shapes ``[B,H,L,D]`` (contiguous unless strides are given)."""
    if mask not in _MASKS:
        raise SdpaValueError(f"SDPA_E_MASK: mask must be one of {sorted(_MASKS)} (got {mask!r})")
    b, hq, lq, dqk = (int(x) for x in q_shape)
    _, hkv, lk, _ = (int(x) for x in k_shape)
    dv = int(v_shape[3])
    d = sdpa_desc_t()
    d.batch, d.heads_q, d.heads_kv, d.len_q, d.len_k, d.dim_qk, d.dim_v = b, hq, hkv, lq, lk, dqk, dv

    def contig(h, l, dd):
        return (h * l * dd, l * dd, dd)

    for name, given, dflt in (("q_stride", q_stride, contig(hq, lq, dqk)),
                              ("k_stride", k_stride, contig(hkv, lk, dqk)),
                              ("v_stride", v_stride, contig(hkv, lk, dv)),
                              ("o_stride", o_stride, contig(hq, lq, dv))):
        arr = getattr(d, name)
        for j, s in enumerate(given if given is not None else dflt):
            arr[j] = int(s)
    d.dtype = int(dtype)
    d.mask = _MASKS[mask]
    d.window = int(window_size) if mask == "window" else int(window_size or 0)
    d.scale = float(1.0 / math.sqrt(dqk)) if scale is None else float(scale)
    d.num_splits = int(num_splits)
    d.row_tile = int(row_tile)
    d.mask_array = int(mask_array)
    for j, st in enumerate(mask_stride):
        d.mask_stride[j] = int(st)
    return d


def pad_mask(mask, dtype=None):
    """Copy a mask array into storage whose rows are padded to 16 bytes.

    Returns a view with the mask's shape (as ``bool`` or ``dtype``) whose key
    rows live in a buffer rounded up to a multiple of 16 bytes, which is the
    layout ``forward(attn_mask=...)`` reads.  Broadcast (size-1) dims stay
    size 1.  This is a preparation step for callers, run once per mask, not
    part of the attention call.
    """
    import torch

    dt = torch.bool if mask.dtype == torch.bool else (dtype or mask.dtype)
    esize = torch.empty((), dtype=dt).element_size()
    lk = mask.shape[-1]
    per = 16 // esize
    lkp = (lk + per - 1) // per * per
    buf = torch.zeros(tuple(mask.shape[:-1]) + (lkp,), dtype=dt, device=mask.device)
    view = buf[..., :lk]
    view.copy_(mask)
    return view


def _mask_layout(attn_mask, q, b, hq, lq, lk):
    """(kind, element strides of (batch, head, query)) of a mask tensor, validated."""
    import torch

    if not isinstance(attn_mask, torch.Tensor):
        raise SdpaValueError("SDPA_E_MASK: attn_mask must be a tensor")
    if attn_mask.device != q.device:
        raise SdpaValueError("SDPA_E_DEVICE: attn_mask must be on the device of q")
    if attn_mask.dtype == torch.bool or attn_mask.dtype == torch.uint8:
        kind = SDPA_MASK_ARRAY_BOOL
    elif attn_mask.dtype == q.dtype:
        kind = SDPA_MASK_ARRAY_ADD
    else:
        raise SdpaValueError("SDPA_E_DTYPE: attn_mask must be bool (True keeps a key) or q's dtype "
                             "(added to the scaled scores)")
    m = attn_mask
    if m.dim() > 4:
        raise SdpaValueError("SDPA_E_SHAPE: attn_mask has at most 4 dims")
    while m.dim() < 4:
        m = m.unsqueeze(0)
    want = (b, hq, lq, lk)
    for j in range(4):
        if m.shape[j] not in (1, want[j]):
            raise SdpaValueError(f"SDPA_E_SHAPE: attn_mask of shape {tuple(attn_mask.shape)} does not "
                                 f"broadcast to [B, Hq, Lq, Lk] = {list(want)}")
    if m.shape[3] != lk:
        raise SdpaValueError("SDPA_E_SHAPE: attn_mask must span all Lk keys in its last dim")
    if lk > 1 and m.stride(3) != 1:
        raise SdpaValueError("SDPA_E_STRIDE: attn_mask must have unit stride in the key dim")
    strides = [m.stride(j) if m.shape[j] > 1 else 0 for j in range(3)]
    esize = m.element_size()
    pad = 16 // esize
    if m.data_ptr() % 16 or any((st * esize) % 16 for st in strides):
        raise SdpaValueError("SDPA_E_STRIDE: attn_mask rows must start on 16-byte boundaries; "
                             "prepare it with pad_mask()")
    # every row is read up to Lk rounded up to 16 bytes
    last = sum(st * (m.shape[j] - 1) for j, st in enumerate(strides)) + (lk + pad - 1) // pad * pad
    if (m.storage_offset() + last) * esize > m.untyped_storage().nbytes():
        raise SdpaValueError("SDPA_E_STRIDE: attn_mask rows must be readable up to Lk rounded up to "
                             "16 bytes; prepare it with pad_mask()")
    return kind, strides


def plan_for(desc: sdpa_desc_t) -> str:
    return sdpa_describe_plan(desc)


def workspace_for(desc: sdpa_desc_t) -> int:
    return sdpa_workspace_bytes(desc)


def forward(q, k, v, *, scale: Optional[float] = None, mask: str = "none", window_size: int = 0,
            attn_mask=None, q_lens=None, kv_lens=None, return_lse: bool = False,
            num_splits: int = 0, row_tile: int = 0,
            out=None, lse_out=None, workspace=None, stream=None
            ) -> Union["torch.Tensor", Tuple["torch.Tensor", "torch.Tensor"]]:  # noqa: F821
    """Fused attention forward on the current HIP device.

    q ``[B,Hq,Lq,Dqk]``, k ``[B,Hkv,Lk,Dqk]``, v ``[B,Hkv,Lk,Dv]`` on one GPU, one
    dtype (float32/float16/bfloat16), unit stride in the head dim.  ``scale``
    defaults to ``1/sqrt(Dqk)``.  ``mask`` is ``"none"``, ``"causal"`` (query
    rows aligned to the last Lq keys) or ``"window"`` (causal plus the last
    ``window_size`` keys).  ``attn_mask`` (optional) broadcasts to
    ``[B,Hq,Lq,Lk]``: a ``bool`` array (or a ``uint8`` one holding only 0
    and 1) keeps the keys where it is true; an array in q's dtype is added
    to the scaled scores.  It applies on top of ``mask``.  Its rows must start
    on 16-byte boundaries and be readable up to Lk rounded up to 16 bytes
    (``pad_mask`` prepares such a copy).  ``q_lens`` / ``kv_lens``
    (optional int32 device tensors ``[B]``) give each batch entry's valid
    queries and keys: entry b's query i sits at key position
    ``i + kv_lens[b] - q_lens[b]``, keys past ``kv_lens[b]`` are never read,
    and rows past ``q_lens[b]`` of the outputs are not written.  Returns ``o`` (and the float32
    log-sum-exp ``[B,Hq,Lq]`` when ``return_lse``).  Validation errors raise
    ``SdpaValueError`` (a ``ValueError``) naming the constraint.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4:
            raise SdpaValueError(f"SDPA_E_SHAPE: {name} must be a 4-D tensor [B, H, L, D]")
        if not t.is_cuda:
            raise SdpaValueError(f"SDPA_E_DEVICE: {name} must be on a GPU; there is no CPU path")
        if t.stride(3) != 1:
            raise SdpaValueError(f"SDPA_E_STRIDE: {name} must have unit stride in the head dim")
    if not (q.dtype == k.dtype == v.dtype):
        raise SdpaValueError("SDPA_E_DTYPE: q, k and v must share one dtype")
    if not (q.device == k.device == v.device):
        raise SdpaValueError("SDPA_E_DEVICE: q, k and v must be on one device")
    dt = _dtype_code(q.dtype)
    b, hq, lq, _ = q.shape
    dv = v.shape[3]
    if out is None:
        out = torch.empty((b, hq, lq, dv), dtype=q.dtype, device=q.device)
    elif out.shape != (b, hq, lq, dv) or out.dtype != q.dtype or out.stride(3) != 1:
        raise SdpaValueError("SDPA_E_SHAPE: out must be [B, Hq, Lq, Dv] in the input dtype")
    kind, mstr = SDPA_MASK_ARRAY_NONE, (0, 0, 0)
    if attn_mask is not None:
        kind, mstr = _mask_layout(attn_mask, q, b, hq, lq, k.shape[2])
    desc = make_desc(q.shape, k.shape, v.shape, dt, scale=scale, mask=mask, window_size=window_size,
                     q_stride=q.stride()[:3], k_stride=k.stride()[:3], v_stride=v.stride()[:3],
                     o_stride=out.stride()[:3], num_splits=num_splits, row_tile=row_tile,
                     mask_array=kind, mask_stride=mstr)
    lse = None
    if return_lse:
        lse = lse_out if lse_out is not None else torch.empty((b, hq, lq), dtype=torch.float32,
                                                              device=q.device)
        if lse.shape != (b, hq, lq) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise SdpaValueError("SDPA_E_SHAPE: lse_out must be contiguous float32 [B, Hq, Lq]")
    nbytes = sdpa_workspace_bytes(desc)
    if nbytes > 0 and (workspace is None or workspace.numel() * workspace.element_size() < nbytes):
        if stream is not None:
            # A workspace allocated here is stream-ordered on torch's current
            # stream only; a caller-chosen stream must bring its own.
            raise SdpaValueError(f"SDPA_E_WORKSPACE: a split plan on an explicit stream needs a "
                                 f"caller workspace of {nbytes} bytes")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if (workspace is not None and nbytes > 0) else 0
    ws_len = workspace.numel() * workspace.element_size() if ws_ptr else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lens = []
    for name, t in (("q_lens", q_lens), ("kv_lens", kv_lens)):
        if t is None:
            lens.append(0)
            continue
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != b
                or not t.is_contiguous() or t.device != q.device):
            raise SdpaValueError(f"SDPA_E_SHAPE: {name} must be a contiguous int32 [B] tensor on q's device")
        lens.append(t.data_ptr())
    with torch.cuda.device(q.device):
        sdpa_forward_varlen(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            attn_mask.data_ptr() if attn_mask is not None else 0, lens[0], lens[1],
                            out.data_ptr(), lse.data_ptr() if lse is not None else 0, ws_ptr, ws_len, stream)
    return (out, lse) if return_lse else out


def backward(q, k, v, o, dout, lse, *, scale: Optional[float] = None, mask: str = "none",
             window_size: int = 0, attn_mask=None, q_lens=None, kv_lens=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None, kv_parts: int = 0):
    """Gradients ``(dq, dk, dv)`` of the fused forward on the current HIP device.

    ``q, k, v`` and ``scale``, ``mask``, ``window_size``, ``attn_mask``,
    ``q_lens``, ``kv_lens`` as given to ``forward``; ``o`` and ``lse`` its
    output and float32 log-sum-exp (``return_lse=True``); ``dout`` the
    upstream gradient, shaped and strided like ``o``.  The mask array is a
    constant (no gradient for it).  With per-batch lengths every gradient
    position past them is 0.  float16 / bfloat16, head dims up to 128.
    Deterministic.  ``kv_parts`` (0: the planner's choice) forces the number
    of row parts each dK/dV key tile is cut into (``desc.num_splits``).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.dim() != 4 or not t.is_cuda or t.stride(3) != 1:
            raise SdpaValueError(f"SDPA_E_SHAPE: {name} must be a 4-D GPU tensor with unit head-dim stride")
        if t.dtype != q.dtype:
            raise SdpaValueError("SDPA_E_DTYPE: q, k, v, o and dout must share one dtype")
    if dout.shape != o.shape or dout.stride() != o.stride():
        raise SdpaValueError("SDPA_E_STRIDE: dout must have o's shape and strides")
    b, hq, lq, _ = q.shape
    if (lse.shape != (b, hq, lq) or lse.dtype != torch.float32 or not lse.is_contiguous()
            or lse.device != q.device):
        raise SdpaValueError("SDPA_E_SHAPE: lse must be the forward's contiguous float32 [B, Hq, Lq]")
    dt = _dtype_code(q.dtype)
    kind, mstr = SDPA_MASK_ARRAY_NONE, (0, 0, 0)
    if attn_mask is not None:
        kind, mstr = _mask_layout(attn_mask, q, b, hq, lq, k.shape[2])
    desc = make_desc(q.shape, k.shape, v.shape, dt, scale=scale, mask=mask, window_size=window_size,
                     q_stride=q.stride()[:3], k_stride=k.stride()[:3], v_stride=v.stride()[:3],
                     o_stride=o.stride()[:3], mask_array=kind, mask_stride=mstr, num_splits=kv_parts)
    outs = []
    for name, given, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if given is None:
            given = torch.empty_strided(like.shape, like.stride(), dtype=like.dtype, device=like.device)
        elif given.shape != like.shape or given.stride() != like.stride() or given.dtype != like.dtype:
            raise SdpaValueError(f"SDPA_E_STRIDE: {name} must have the shape, strides and dtype of its input")
        outs.append(given)
    nbytes = sdpa_backward_workspace_bytes(desc)
    if workspace is None or workspace.numel() * workspace.element_size() < nbytes:
        if stream is not None:
            raise SdpaValueError(f"SDPA_E_WORKSPACE: the backward pass on an explicit stream needs a caller "
                                 f"workspace of {nbytes} bytes")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    lens = []
    for name, t in (("q_lens", q_lens), ("kv_lens", kv_lens)):
        if t is None:
            lens.append(0)
            continue
        if (not isinstance(t, torch.Tensor) or t.dtype != torch.int32 or t.dim() != 1 or t.shape[0] != b
                or not t.is_contiguous() or t.device != q.device):
            raise SdpaValueError(f"SDPA_E_SHAPE: {name} must be a contiguous int32 [B] tensor on q's device")
        lens.append(t.data_ptr())
    with torch.cuda.device(q.device):
        sdpa_backward_varlen(desc, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             attn_mask.data_ptr() if attn_mask is not None else 0, lens[0], lens[1],
                             o.data_ptr(), dout.data_ptr(), lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                             outs[2].data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             stream)
    return tuple(outs)
