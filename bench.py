#!/usr/bin/env python3
"""Benchmark of the fused SDPA forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--sweep]

A step is one ``sdpa_forward`` call (validate + plan on the host, the
attention kernel, and the split combine when the plan splits) over one batch
of seeded synthetic N(0, 1) inputs already resident in HBM.  The default
workload is the GQA decode with asymmetric head dims at its largest KV set:
B=1, Hq=64, Hkv=8, Lq=1, Lk=32768, Dqk=192, Dv=128, bfloat16, causal (the
query at the last position).  Its metric is the algorithmic KV bandwidth:
bytes of Q + K + V + O per step over the step time.

The KV set (168 MB) fits in the 256 MB Infinity Cache, so consecutive steps
rotate over enough identical copies of K/V (> 2 x 256 MB in total) that every
step streams its K/V from HBM, not from the cache.

Printed: ONE JSON line with the metric, plus ``roofline`` (the algorithmic
bytes per call over the call's device time, attention kernel plus the split
combine, measured with HIP events recorded on the launch stream by the
library's profiling hook; mean, median, p10 and p90 over at least 40 calls)
and ``cpu_baseline`` (the float64 oracle timed on the host cores).  The
default line also carries ``prefill``, the other half of the metric: the
causal D=256 layer at L=32768 (Hq=16, Hkv=2) timed the same way with its own
roofline (algorithmic flops over MFMA peak) and oracle baseline, and under
``configs`` the encoder, vision and windowed D=256 prefill workloads (10
warm-up and 40 timed calls each, median with p10 and p90).

``--sweep`` additionally times every shape of the table below (the five
workloads, then explicit mask arrays beside the same shapes without one) and
writes a table (stderr) and JSON (``--sweep-out``).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SDPA prefill TFLOP/s & decode KV GB/s on 1 MI355X, % of roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA16_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16 MFMA
FP32_PEAK_TFLOPS = 157.3     # fp32 matrix
INFINITY_CACHE = 256 << 20
ES = {"f32": 4, "f16": 2, "bf16": 2}

# Fused decode on the pages: 64 query / 8 KV heads, Lk=32768, bf16, 728 us on
# Apple M3 Ultra (mlx PR #3637 "Enable fused SDPA vector kernel for asymmetric
# Q/V head dims (192, 128)", second benchmark table).  Context, not a target.
PAGES_DECODE_US = {(4, 256): 218, (4, 1024): 217, (4, 4096): 255, (4, 8192): 305, (4, 16384): 382,
                   (4, 32768): 599, (8, 256): 207, (8, 1024): 222, (8, 4096): 288, (8, 8192): 358,
                   (8, 16384): 444, (8, 32768): 728}


def pages_shape(s):
    """True for the decode shapes the pages time (B=1, Hq=64, Lq=1, Dqk=192,
    Dv=128, bf16, one of their Hkv / Lk), the only ones ``vs_baseline`` may use."""
    return (s["b"], s["hq"], s["lq"], s["dqk"], s["dv"], s["dtype"]) == (1, 64, 1, 192, 128, "bf16") and \
        (s["hkv"], s["lk"]) in PAGES_DECODE_US and s.get("arr") is None and not s.get("varlen")


def shape(name, b, hq, hkv, lq, lk, dqk, dv, dtype, mask, window, seed, arr=None, arr_window=0,
          varlen=False, bwd=False):
    """One benchmark shape.  ``arr`` names an explicit mask array given on top
    of the mode: "window_bool" (an [Lq, Lk] boolean band of the last
    ``arr_window`` keys, what callers build without a window mode),
    "bias_add" (an [Lq, Lk] additive N(0, 1) bias) or "pad_bool" (a
    [B, 1, 1, Lk] key-padding mask).  ``varlen`` passes the same per-entry
    key lengths as "pad_bool" uses as kv_lens instead.  ``bwd`` times the
    backward pass (dQ, dK, dV) of the shape instead of the forward."""
    return dict(name=name, b=b, hq=hq, hkv=hkv, lq=lq, lk=lk, dqk=dqk, dv=dv, dtype=dtype,
                mask=mask, window=window, seed=seed, arr=arr, arr_window=arr_window, varlen=varlen, bwd=bwd)


def all_shapes():
    """Every shape of the five workloads (seeds 1000 * workload + index), then
    the mask array shapes (seeds 6000 + index)."""
    out = [shape("tiny_f32", 1, 4, 4, 128, 128, 64, 64, "f32", "none", 0, 1000)]
    lks = [256, 1024, 4096, 8192, 16384, 32768]
    for j, hkv in enumerate((4, 8)):
        for i, lk in enumerate(lks):
            out.append(shape(f"decode_hkv{hkv}_lk{lk}", 1, 64, hkv, 1, lk, 192, 128, "bf16", "causal", 0,
                             2000 + i + j * len(lks)))
    lqs = [1, 2, 4, 8, 12, 16, 24, 32, 48, 64]
    for j, lk in enumerate((16384, 32768)):
        for i, lq in enumerate(lqs):
            out.append(shape(f"verify_lk{lk}_lq{lq}", 1, 32, 8, lq, lk, 128, 128, "f16", "none", 0,
                             3000 + i + j * len(lqs)))
    out.append(shape("encoder_h20_l1500_d64", 1, 20, 20, 1500, 1500, 64, 64, "bf16", "none", 0, 4000))
    out.append(shape("vision_h16_l1024_d72", 1, 16, 16, 1024, 1024, 72, 72, "bf16", "none", 0, 4001))
    out.append(shape("vision_h16_l4096_d72", 1, 16, 16, 4096, 4096, 72, 72, "bf16", "none", 0, 4002))
    for i, L in enumerate((2048, 4096, 8192)):
        out.append(shape(f"window_l{L}_d256", 1, 16, 8, L, L, 256, 256, "bf16", "window", 1024, 5000 + i))
    out.append(shape("causal_l32768_d256", 1, 16, 2, 32768, 32768, 256, 256, "bf16", "causal", 0, 5003))
    # explicit mask arrays, each beside the same shape without one
    out.append(shape("maskarr_window_bool_l4096_d256", 1, 16, 8, 4096, 4096, 256, 256, "bf16", "none", 0,
                     6000, arr="window_bool", arr_window=1024))
    out.append(shape("causal_l4096_d128", 1, 16, 16, 4096, 4096, 128, 128, "bf16", "causal", 0, 6001))
    out.append(shape("maskarr_bias_add_causal_l4096_d128", 1, 16, 16, 4096, 4096, 128, 128, "bf16", "causal", 0,
                     6001, arr="bias_add"))
    out.append(shape("decode_b4_hkv8_lk8192_d128", 4, 32, 8, 1, 8192, 128, 128, "bf16", "none", 0, 6002))
    out.append(shape("maskarr_pad_decode_b4_hkv8_lk8192_d128", 4, 32, 8, 1, 8192, 128, 128, "bf16", "none", 0,
                     6002, arr="pad_bool"))
    # head dim 512 (zero-padded MFMA dims above 256 land here too)
    out.append(shape("causal_l8192_d512", 1, 16, 2, 8192, 8192, 512, 512, "bf16", "causal", 0, 8000))
    out.append(shape("decode_d512_hkv8_lk16384", 1, 32, 8, 1, 16384, 512, 512, "bf16", "causal", 0, 8001))
    # backward pass, beside the forward of the same shape (causal_l4096_d128)
    out.append(shape("bwd_causal_l4096_d128", 1, 16, 16, 4096, 4096, 128, 128, "bf16", "causal", 0, 6001, bwd=True))
    # the same layer with grouped queries (4 query heads per KV head)
    out.append(shape("bwd_causal_gqa_l4096_d128", 1, 32, 8, 4096, 4096, 128, 128, "bf16", "causal", 0, 6003,
                     bwd=True))
    # per-entry key lengths, beside the same lengths as a padding mask
    out.append(shape("decode_b8_hkv8_lk8192_d128", 8, 32, 8, 1, 8192, 128, 128, "bf16", "none", 0, 7000))
    out.append(shape("maskarr_pad_decode_b8_hkv8_lk8192_d128", 8, 32, 8, 1, 8192, 128, 128, "bf16", "none", 0,
                     7000, arr="pad_bool"))
    out.append(shape("varlen_decode_b8_hkv8_lk8192_d128", 8, 32, 8, 1, 8192, 128, 128, "bf16", "none", 0, 7000,
                     varlen=True))
    return out


SHAPES = {s["name"]: s for s in all_shapes()}
DEFAULT = "decode_hkv8_lk32768"


def visible_pairs(lq, lk, mask, window):
    """Visible (query, key) pairs of one head, closed form (bottom-right aligned masks)."""
    off = lk - lq
    if mask == "none":
        return lq * lk
    if mask == "causal":
        return lq * (lq + 1) // 2 + lq * off
    w = window
    # row i sees min(w, i + off + 1) keys
    first_full = max(0, w - 1 - off)  # rows i >= first_full see w keys
    if first_full >= lq:
        return lq * (lq + 1) // 2 + lq * off
    partial = first_full * (first_full + 1) // 2 + first_full * off
    return partial + (lq - first_full) * w


def row_visible(i, s):
    """Keys visible to query row i (bottom-right aligned masks)."""
    pos = s["lk"] - s["lq"] + i
    if s["mask"] == "none":
        return s["lk"]
    if s["mask"] == "causal":
        return pos + 1
    return min(s["window"], pos + 1)


def mask_array_bytes(s):
    """Bytes of the distinct elements of the workload's mask array (0 without one)."""
    arr = s.get("arr")
    if arr is None:
        return 0
    if arr == "pad_bool":
        return s["b"] * s["lk"]
    return s["lq"] * s["lk"] * (1 if arr == "window_bool" else ES[s["dtype"]])


def kv_lengths(s):
    """Per-entry key lengths of a shape with a padding mask or varlen (else None)."""
    if s.get("arr") != "pad_bool" and not s.get("varlen"):
        return None
    from scaled_dot_product_fwd_amd.synth import lengths

    return [int(x) for x in lengths(s["b"], s["lk"] // 4, s["lk"], s["seed"] + 3)]


def work(s):
    """(algorithmic flops, algorithmic bytes) of one call.

    With a mask array every pair the mode keeps is evaluated: the array is
    data, so which of its blocks are empty is not known ahead of the call.
    Its distinct elements count once in the bytes.  With per-entry lengths
    only each entry's valid keys count.
    """
    es = ES[s["dtype"]]
    d = s["dqk"] + s["dv"]
    if s.get("bwd"):
        # recompute S once, then dP, dV, dQ, dK: 2 (3 Dqk + 2 Dv) per visible pair;
        # read q, k, v, o, dO (+ lse), write dq, dk, dv
        pairs = visible_pairs(s["lq"], s["lk"], s["mask"], s["window"])
        flops = 2 * s["b"] * s["hq"] * (3 * s["dqk"] + 2 * s["dv"]) * pairs
        nbytes = es * s["b"] * (s["hq"] * s["lq"] * 2 * d + s["hkv"] * s["lk"] * 2 * d) + 4 * s["b"] * s["hq"] * s["lq"]
        return flops, nbytes
    if s.get("varlen"):
        kl = kv_lengths(s)
        pairs = sum(visible_pairs(s["lq"], n, s["mask"], s["window"]) for n in kl)
        flops = 2 * s["hq"] * d * pairs
        nbytes = es * (s["b"] * s["hq"] * s["lq"] * d + s["hkv"] * sum(kl) * d)
        return flops, nbytes
    pairs = visible_pairs(s["lq"], s["lk"], s["mask"], s["window"])
    flops = 2 * s["b"] * s["hq"] * d * pairs
    nbytes = es * s["b"] * (s["hq"] * s["lq"] * d + s["hkv"] * s["lk"] * d)
    return flops, nbytes + mask_array_bytes(s)


def make_mask_array(s):
    """CPU mask array of the workload (None without one)."""
    import torch

    from scaled_dot_product_fwd_amd.synth import additive_mask, padding_mask

    arr = s.get("arr")
    if arr is None:
        return None
    if arr == "pad_bool":
        return padding_mask(s["b"], s["lk"], s["seed"] + 3, min_len=s["lk"] // 4)  # lengths as kv_lengths(s)
    if arr == "bias_add":
        return additive_mask((s["lq"], s["lk"]), s["seed"] + 3, torch.bfloat16 if s["dtype"] == "bf16" else
                             (torch.float16 if s["dtype"] == "f16" else torch.float32), sigma=1.0, minus_inf=0.0)
    # band of the last arr_window key positions up to the query's own (rows
    # aligned to the last Lq keys)
    pos = torch.arange(s["lq"])[:, None] + (s["lk"] - s["lq"])
    key = torch.arange(s["lk"])[None, :]
    return (key <= pos) & (key > pos - s["arr_window"])


def bound(s):
    """'hbm' for decode-shaped calls (arithmetic intensity below the ridge), else 'mfma'."""
    flops, nbytes = work(s)
    peak = FP32_PEAK_TFLOPS if s["dtype"] == "f32" else MFMA16_PEAK_TFLOPS
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    return "hbm" if flops / nbytes < ridge else "mfma"


class HipEvents:
    """hipEvent_t pairs through the HIP runtime torch already loaded.

    The events are timing-only (hipEventDisableSystemFence): recording them
    does not write back and invalidate the caches, which would both inflate
    the bracketed interval and slow the kernel after them.  They are read
    only after a full device synchronisation.
    """

    TIMING_ONLY = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.start, self.stop = [], []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            if (self.hip.hipEventCreateWithFlags(ctypes.byref(a), self.TIMING_ONLY)
                    or self.hip.hipEventCreateWithFlags(ctypes.byref(b), self.TIMING_ONLY)):
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.start.append(a.value)
            self.stop.append(b.value)

    def record(self, ev, stream):
        if self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]):
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self):
        for e in self.start + self.stop:
            self.hip.hipEventDestroy(e)


class BwdRunner:
    """Pre-built inputs (q, k, v, the forward's o and lse, dO), outputs and
    workspace for repeated raw backward calls.  The HIP events bracket the
    whole call (its three kernels) on the launch stream."""

    def __init__(self, s):
        import torch

        import scaled_dot_product_fwd_amd as sdpa
        from scaled_dot_product_fwd_amd.synth import DTYPES, default_scale, make_qkv, randn

        self.s = s
        self.sdpa = sdpa
        dt = DTYPES[s["dtype"]]
        dev = torch.device("cuda", 0)
        q, k, v = make_qkv(s["b"], s["hq"], s["hkv"], s["lq"], s["lk"], s["dqk"], s["dv"], dt, s["seed"])
        do = randn((s["b"], s["hq"], s["lq"], s["dv"]), s["seed"] + 3, dt)
        self.cpu = (q, k, v, do)
        self.scale = default_scale(s["dqk"])
        self.q, self.k, self.v, self.do = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
        self.o, self.lse = sdpa.forward(self.q, self.k, self.v, scale=self.scale, mask=s["mask"],
                                        window_size=s["window"], return_lse=True)
        self.g = [torch.empty_like(x) for x in (self.q, self.k, self.v)]
        self.desc = sdpa.make_desc(self.q.shape, self.k.shape, self.v.shape, sdpa._dtype_code(dt),
                                   scale=self.scale, mask=s["mask"], window_size=s["window"])
        self.plan = "backward: prep + dq (128-row tiles) + dk/dv (128-key tiles)"
        self.ws_bytes = sdpa.sdpa_backward_workspace_bytes(self.desc)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev).cuda_stream
        self.nsets = 1
        lib = sdpa.load()
        self._bwd = lib.sdpa_backward
        self._descref = ctypes.byref(self.desc)
        self._args = (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.o.data_ptr(),
                      self.do.data_ptr(), self.lse.data_ptr(), self.g[0].data_ptr(), self.g[1].data_ptr(),
                      self.g[2].data_ptr(), self.ws.data_ptr(), self.ws_bytes, self.stream)

    def step(self, i, events=None, j=None):
        if events is not None:
            events.record(events.start[j], self.stream)
        rc = self._bwd(self._descref, *self._args)
        if events is not None:
            events.record(events.stop[j], self.stream)
        if rc:
            self.sdpa._lib.check(rc)


class Runner:
    """Pre-built descriptor, buffers and workspace for repeated raw C calls."""

    def __init__(self, s, kv_bytes_floor=0):
        import torch

        import scaled_dot_product_fwd_amd as sdpa
        from scaled_dot_product_fwd_amd.synth import DTYPES, default_scale, make_qkv

        self.s = s
        self.sdpa = sdpa
        dt = DTYPES[s["dtype"]]
        dev = torch.device("cuda", 0)
        q, k, v = make_qkv(s["b"], s["hq"], s["hkv"], s["lq"], s["lk"], s["dqk"], s["dv"], dt, s["seed"])
        self.cpu = (q, k, v)
        self.scale = default_scale(s["dqk"])
        self.q = q.to(dev)
        kd, vd = k.to(dev), v.to(dev)
        set_bytes = (kd.numel() + vd.numel()) * kd.element_size()
        nsets = 1
        if kv_bytes_floor:
            nsets = max(1, min(64, math.ceil(kv_bytes_floor / set_bytes)))
        self.kv = [(kd, vd)] + [(kd.clone(), vd.clone()) for _ in range(nsets - 1)]
        self.nsets = nsets
        self.o = torch.empty((s["b"], s["hq"], s["lq"], s["dv"]), dtype=dt, device=dev)
        self.lse = torch.empty((s["b"], s["hq"], s["lq"]), dtype=torch.float32, device=dev)
        self.mask_cpu = make_mask_array(s)
        kind, mstr, self.mask = sdpa.SDPA_MASK_ARRAY_NONE, (0, 0, 0), None
        if self.mask_cpu is not None:
            self.mask = sdpa.pad_mask(self.mask_cpu.to(dev))
            kind, mstr = sdpa._mask_layout(self.mask, self.q, s["b"], s["hq"], s["lq"], s["lk"])
        self.desc = sdpa.make_desc(self.q.shape, kd.shape, vd.shape, sdpa._dtype_code(dt), scale=self.scale,
                                   mask=s["mask"], window_size=s["window"], mask_array=kind, mask_stride=mstr,
                                   num_splits=s.get("num_splits", 0), row_tile=s.get("row_tile", 0))
        self.plan = sdpa.sdpa_describe_plan(self.desc)
        self.ws_bytes = sdpa.sdpa_workspace_bytes(self.desc)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream(dev).cuda_stream
        self.kv_lens = None
        if s.get("varlen"):
            self.kv_lens = torch.tensor(kv_lengths(s), dtype=torch.int32, device=dev)
        lib = sdpa.load()
        self._fwd = lib.sdpa_forward_varlen
        self._prof = lib.sdpa_set_profile_events
        self._descref = ctypes.byref(self.desc)
        mptr = self.mask.data_ptr() if self.mask is not None else None
        kvl = self.kv_lens.data_ptr() if self.kv_lens is not None else None
        self._args = [(self.q.data_ptr(), k_.data_ptr(), v_.data_ptr(), mptr, None, kvl, self.o.data_ptr(),
                       self.lse.data_ptr(), self.ws.data_ptr() if self.ws_bytes else None, self.ws_bytes,
                       self.stream)
                      for k_, v_ in self.kv]

    def step(self, i, events=None, j=None):
        if events is not None:
            self._prof(events.start[j], events.stop[j])
        rc = self._fwd(self._descref, *self._args[i % self.nsets])
        if rc:
            self.sdpa._lib.check(rc)

    def output(self):
        return self.o, self.lse


# Every EVENT_EVERY-th timed step records the call's HIP events: two event
# packets around a call cost ~2 us of queue time per step (measured: decode
# step 36.3 us with events on every step, 34.3 us without, 34.6 us with every
# 4th), so sampling keeps the measurement from inflating the step time it
# sits in.
EVENT_EVERY = 4
# Kernel-time samples per workload, as in mlx issue #3826 (report: 10 warm-up
# calls, then 40 timed ones).
MIN_SAMPLES = 40


def time_steps(r, steps, warmup, event_every=EVENT_EVERY, min_samples=MIN_SAMPLES):
    """Warm up, then time exactly `steps` steps; returns (ms_per_step, kernel_ms list).

    The device time of a call (attention kernel plus the split combine, when
    the plan splits) is taken with HIP events recorded on its stream around
    the call in steps 0, event_every, 2 event_every, ... of the timed region.
    When those are fewer than ``min_samples``, the calls right after the
    timed region (same inputs, same rotation, every call sampled) add the
    rest, outside the clock of ``ms_per_step``.
    """
    import torch

    sampled = list(range(0, steps, event_every))
    extra = max(0, min_samples - len(sampled))
    ev = HipEvents(len(sampled) + extra)
    for i in range(warmup):
        r.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % event_every == 0:
            r.step(i, ev, i // event_every)
        else:
            r.step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for n in range(extra):
        r.step(steps + n, ev, len(sampled) + n)
    torch.cuda.synchronize()
    kms = [ev.elapsed_ms(n) for n in range(len(sampled) + extra)]
    ev.close()
    return (t1 - t0) * 1e3 / steps, kms


def cpu_baseline(s, runner, budget_s=12.0):
    """The float64 oracle on the host cores, on a bounded sample of the workload.

    Whole KV groups (all query heads sharing one KV head) are run one after
    another until the time budget is spent; when even one group would blow the
    budget, evenly spaced query rows are recomputed one by one instead.  The
    work done is scaled to the metric's unit.  The oracle's results for the
    sample are also compared with the GPU's output of the same inputs (the
    runner's last call): ``max_abs_err`` holds max |gpu - oracle| over the
    sample (o and lse; for the backward dQ, and dK, dV where one query head
    is its KV head's whole gradient).
    """
    import numpy as np
    from oracle import sdpa_bwd_ref, sdpa_ref, sdpa_ref_rows, sdpa_ref_varlen

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    q, k, v = runner.cpu[:3]
    g = s["hq"] // s["hkv"]
    flops, nbytes = work(s)
    group_flops = flops / s["hkv"]
    t_total, frac, sample = 0.0, 0.0, ""
    err = {}

    def note(key, got, ref):
        d = np.abs(np.asarray(got, dtype=np.float64) - ref)
        # rows that see no key: lse = -inf on both sides counts as equal
        d = np.where(np.isinf(ref) & (np.asarray(got, dtype=np.float64) == ref), 0.0, d)
        err[key] = max(err.get(key, 0.0), float(d.max()) if d.size else 0.0)

    if s.get("bwd"):
        gq, gk, gv = (x.float().cpu().numpy() for x in runner.g)
    else:
        o_gpu = runner.o.float().cpu().numpy()
        lse_gpu = runner.lse.cpu().numpy()
    if s.get("bwd"):
        # whole query heads (with their KV head) until the budget is spent
        do = runner.cpu[3]
        heads = 0
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < budget_s and heads < s["b"] * s["hq"]:
            bi, h = divmod(heads, s["hq"])
            t0 = time.perf_counter()
            rq, rk, rv = sdpa_bwd_ref(q[bi:bi + 1, h:h + 1], k[bi:bi + 1, h // g:h // g + 1],
                                      v[bi:bi + 1, h // g:h // g + 1], do[bi:bi + 1, h:h + 1], runner.scale,
                                      s["mask"], s["window"])
            t_total += time.perf_counter() - t0
            note("dq", gq[bi:bi + 1, h:h + 1], rq)
            if g == 1:
                note("dk", gk[bi:bi + 1, h:h + 1], rk)
                note("dv", gv[bi:bi + 1, h:h + 1], rv)
            heads += 1
        frac = heads / (s["b"] * s["hq"])
        sample = f"{heads} query heads' gradients ({frac:.3f} of one step)"
    elif group_flops < 20e9 * budget_s:  # one group fits the budget at a modest 20 GFLOP/s
        heads = 0
        t_start = time.perf_counter()
        while time.perf_counter() - t_start < budget_s and heads < 50 * s["hq"]:
            kvh = (heads // g) % s["hkv"]
            hs = slice(kvh * g, (kvh + 1) * g)
            t0 = time.perf_counter()
            if s.get("varlen"):
                ro, rl = sdpa_ref_varlen(q[:, hs], k[:, kvh:kvh + 1], v[:, kvh:kvh + 1], runner.scale, s["mask"],
                                         s["window"], kv_lens=kv_lengths(s))
            else:
                ro, rl = sdpa_ref(q[:, hs], k[:, kvh:kvh + 1], v[:, kvh:kvh + 1], runner.scale, s["mask"],
                                  s["window"], mask_arr=runner.mask_cpu)
            t_total += time.perf_counter() - t0
            note("o", o_gpu[:, hs], ro)
            note("lse", lse_gpu[:, hs], rl)
            heads += g
        frac = heads / s["hq"]
        sample = f"{heads} query heads in whole KV groups ({frac:.2f} of one step)"
    else:
        rows_per_head = s["lq"]
        picks, n = [], 0
        stride = max(1, (s["hq"] * rows_per_head) // 4096)
        for t in range(0, s["hq"] * rows_per_head, stride):
            picks.append((0, t // rows_per_head, t % rows_per_head))
        done_flops = 0
        t_start = time.perf_counter()
        for n0 in range(0, len(picks), 64):
            chunk = picks[n0:n0 + 64]
            t0 = time.perf_counter()
            ro, rl = sdpa_ref_rows(q, k, v, runner.scale, s["mask"], s["window"], chunk, mask_arr=runner.mask_cpu,
                                   kv_lens=kv_lengths(s) if s.get("varlen") else None)
            t_total += time.perf_counter() - t0
            idx = tuple(np.array(chunk).T)
            note("o", o_gpu[idx], ro)
            note("lse", lse_gpu[idx], rl)
            for (_, _, i) in chunk:
                done_flops += 2 * (s["dqk"] + s["dv"]) * row_visible(i, s)
            n += len(chunk)
            if time.perf_counter() - t_start > budget_s:
                break
        frac = done_flops / flops
        sample = f"{n} evenly spaced query rows recomputed one by one ({frac:.2e} of one step)"
    sec_per_step = t_total / frac
    if bound(s) == "hbm":
        value, unit = nbytes / sec_per_step / 1e9, "GB/s"
    else:
        value, unit = flops / sec_per_step / 1e12, "TFLOP/s"
    return {"value": round(value, 6), "unit": unit, "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{sample} of the same workload, float64 numpy, {t_total:.1f} s",
            "max_abs_err": {k_: float(f"{e:.3g}") for k_, e in err.items()}}


def cpu_model():
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def kernel_source_hash(name):
    """Fingerprint of what a counter run of workload ``name`` measured: every
    device-side source (kernels, launchers, argument set-up; the host planner
    is left out) plus the plan the planner makes for the workload, so a
    planner change that alters this workload's launch also invalidates it."""
    import scaled_dot_product_fwd_amd as sdpa
    from scaled_dot_product_fwd_amd.synth import DTYPES

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "scaled_dot_product_fwd_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f == "plan.cpp":
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    s = SHAPES[name]
    desc = sdpa.make_desc((s["b"], s["hq"], s["lq"], s["dqk"]), (s["b"], s["hkv"], s["lk"], s["dqk"]),
                          (s["b"], s["hkv"], s["lk"], s["dv"]), sdpa._dtype_code(DTYPES[s["dtype"]]),
                          mask=s["mask"], window_size=s["window"])
    h.update(sdpa.sdpa_describe_plan(desc).encode())
    return h.hexdigest()[:16]


def traffic_from_profiles(name):
    """HBM bytes per launch from the committed counter summary, if it matches the sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(name):
        return None
    return t.get("hbm_bytes_per_launch")


def context_rates():
    """What the part delivers to plain library code, beside the quoted peaks:
    a device-to-device copy of 1 GiB (read + written bytes over its time) and
    a 8192^3 bfloat16 matrix product through torch (hipBLASLt), each the
    median of 20 runs after 3 warm-up, HIP events on the current stream.
    Context only: the roofline fractions stay against the quoted peaks."""
    import torch

    def med(fn, n=20):
        for _ in range(3):
            fn()
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[n // 2]

    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    copy_ms = med(lambda: dst.copy_(src))
    del src, dst
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    gemm_ms = med(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * (1 << 30) / (copy_ms * 1e-3) / 1e9, 1),
            "gemm_bf16_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "what": "1 GiB device copy (read + write bytes) and an 8192^3 bf16 torch.matmul (hipBLASLt), "
                    "median of 20; context beside the quoted 8 TB/s and 2.5 PFLOP/s"}


def calibration_copy(mib):
    """A plain device copy of known size (float32 ``dst = src * 1``), run three
    times, so that a counter run over this process can scale its HBM byte
    counters by what they read for a known number of bytes."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def summarize_pmc(fetch_dir, write_dir, name, copy_mib, commands):
    """Reduce two ``rocprofv3 --pmc`` runs (FETCH_SIZE, WRITE_SIZE) of
    ``bench.py --workload NAME --calibrate-copy-mib M`` to HBM bytes per launch
    of the attention kernel: each counter's KiB per dispatch, averaged over the
    attention dispatches, times (known bytes / counter bytes) of the copy."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] != counter:
                        continue
                    vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    def pick(vals, needle):
        rows = [(k, v) for k, v in vals.items() if needle(k)]
        if not rows:
            raise SystemExit(f"no dispatch matched in {sorted(vals)[:8]}")
        k, v = max(rows, key=lambda kv: len(kv[1]))
        return k, v

    copy_bytes = 2 * copy_mib * (1 << 20)  # read once, written once
    _, inst = instance_of(SHAPES[name])
    out = {"workload": name, "kernel_source_hash": kernel_source_hash(name), "commands": commands,
           "copy": {"kernel": "float32 dst = src * 1", "bytes_read": copy_bytes // 2,
                    "bytes_written": copy_bytes // 2}}
    total, comb_total, fetch_raw = 0.0, 0.0, 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = per_kernel(d, counter)
        kname, kv = pick(vals, lambda k: "attn_fwd_kernel" in k and inst in k)
        cname, cv = pick(vals, lambda k: "elementwise" in k and "Mul" in k)
        cv = [x for x in cv if x > 0.25 * copy_bytes / 2 / 1024] or cv
        k_kib = sum(kv) / len(kv)
        c_kib = sum(cv) / len(cv)
        factor = (copy_bytes / 2) / (c_kib * 1024)
        out[counter] = {"attention_kib_per_dispatch": round(k_kib, 1), "dispatches": len(kv),
                        "copy_kib_per_dispatch": round(c_kib, 1), "scale": round(factor, 4)}
        # the split combine of the same calls (partials read, output written)
        comb = [v for k, v in vals.items() if "combine_kernel" in k]
        if comb:
            cb = max(comb, key=len)
            out[counter]["combine_kib_per_dispatch"] = round(sum(cb) / len(cb), 1)
            comb_total += sum(cb) / len(cb) * 1024 * factor
        out["kernel"] = kname
        total += k_kib * 1024 * factor
        if counter == "FETCH_SIZE":
            fetch_raw = k_kib * 1024
    s = SHAPES[name]
    out["hbm_bytes_per_launch"] = int(total)
    out["algorithmic_bytes_per_launch"] = work(s)[1]
    out["ratio_to_algorithmic"] = round(total / work(s)[1], 4)
    if comb_total:
        out["combine_hbm_bytes_per_launch"] = int(comb_total)
        out["call_ratio_to_algorithmic"] = round((total + comb_total) / work(s)[1], 4)
    # The copy calibrates the scale with ordinary loads.  The attention
    # kernel loads K and V by LDS DMA; that the same scale holds for them
    # follows from a lower bound: every K/V byte must be read at least once,
    # so unscaled FETCH_SIZE below the K/V bytes means the counter sees the
    # same fraction of these loads.
    kv_bytes = 2 * s["b"] * s["hkv"] * s["lk"] * (s["dqk"] + s["dv"])
    out["scale_check"] = {"fetch_unscaled_bytes": int(fetch_raw), "kv_bytes_read_at_least_once": kv_bytes,
                          "unscaled_below_minimum": bool(fetch_raw < kv_bytes)}
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def instance_of(s):
    """(plan string, template-argument prefix of the attention kernel instance
    the plan launches), e.g. "BF16, 192, 128, 1, 4, 32", to pick the
    workload's own dispatches out of a trace."""
    import scaled_dot_product_fwd_amd as sdpa
    from scaled_dot_product_fwd_amd.synth import DTYPES

    desc = sdpa.make_desc((s["b"], s["hq"], s["lq"], s["dqk"]), (s["b"], s["hkv"], s["lk"], s["dqk"]),
                          (s["b"], s["hkv"], s["lk"], s["dv"]), sdpa._dtype_code(DTYPES[s["dtype"]]),
                          mask=s["mask"], window_size=s["window"])
    plan = sdpa.sdpa_describe_plan(desc)
    pl = dict(tok.split("=", 1) for tok in plan.split())
    nwq, nwk = (int(x) for x in pl["waves"].split("x")[:2])
    inst = "{}, {}, {}, {}, {}, {}".format({"bf16": "BF16", "f16": "F16", "f32": "F32"}[s["dtype"]],
                                           pl["dqk"].split("->")[1], pl["dv"].split("->")[1], nwq, nwk,
                                           int(pl["block_keys"]) // nwk)
    return plan, inst


def summarize_trace(trace_dir, name, command):
    """Reduce a ``rocprofv3 --kernel-trace --stats --output-format csv`` run of
    ``bench.py --workload NAME`` to profiles/NAME_kernel_stats.md: calls and
    average / min / max duration per kernel, the call's device time (the
    attention kernel plus the combine, when the plan splits) and the roofline
    fraction it gives."""
    import csv
    import glob

    s = SHAPES[name]
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {trace_dir}")
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"])))
    flops, nbytes = work(s)
    plan, inst = instance_of(s)
    span_line = ""
    if s.get("bwd"):
        # a backward call is the prep, dQ and dK/dV kernels (the forward that
        # produces o and lse runs once, outside the timed calls); dQ and dK/dV
        # overlap on two streams, so the call is the span from the prep's
        # start to the last of the call's kernels to end, per call in the trace
        parts = [[r for r in rows if k in r[0]]
                 for k in ("bwd_prep_kernel", "bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_kvsum_kernel")]
        call_name = " + ".join(f"`{p[0][0]}`" for p in parts if p)
        spans = bwd_call_spans(trace_dir)
        call_ns = sum(spans) / len(spans) if spans else sum(p[0][2] for p in parts if p)
        span_line = (f"Call spans (prep start to the last kernel's end, {len(spans)} calls): mean {call_ns:.0f} ns, "
                     f"min {min(spans):.0f} ns; the kernels' averages add up to "
                     f"{sum(p[0][2] for p in parts if p):.0f} ns because dQ and dK/dV overlap.") if spans else ""
        plan = ("backward: bwd_prep, then bwd_dq (128-row tiles, second stream) beside bwd_dkdv "
                "(128-key tiles)")
    else:
        # the workload's own instance (a default run also times the prefill workloads)
        attn = [r for r in rows if "attn_fwd_kernel" in r[0] and inst in r[0]]
        comb = [r for r in rows if "combine_kernel" in r[0]] if " splits=1 " not in plan else []
        call_ns = (attn[0][2] if attn else 0.0) + (comb[0][2] if comb else 0.0)
        call_name = f"`{attn[0][0] if attn else '?'}`" + (" + combine kernel" if comb else "")
    if bound(s) == "hbm":
        rate = nbytes / (call_ns * 1e-9) / 1e9
        frac = rate / HBM_PEAK_GBS
        work_line = f"Algorithmic bytes per call: {nbytes:,} B; by rocprof {rate:.0f} GB/s = {100 * frac:.1f}% of 8 TB/s."
    else:
        peak = FP32_PEAK_TFLOPS if s["dtype"] == "f32" else MFMA16_PEAK_TFLOPS
        rate = flops / (call_ns * 1e-9) / 1e12
        frac = rate / peak
        work_line = (f"Algorithmic flops per call: {flops:,}; by rocprof {rate:.1f} TFLOP/s = "
                     f"{100 * frac:.1f}% of {peak:.0f} TFLOP/s.")
    out = [f"# Kernel trace: {name}", "",
           f"B={s['b']} Hq={s['hq']} Hkv={s['hkv']} Lq={s['lq']} Lk={s['lk']} Dqk={s['dqk']} Dv={s['dv']} "
           f"{s['dtype']} mask={s['mask']}" + (f"({s['window']})" if s["window"] else ""), "",
           "Command (from /tmp with TMPDIR=/tmp; `$R` is the repository root):", "", "    " + command, "",
           f"Plan: {plan}", "",
           "| kernel | calls | avg ns | min ns | max ns |", "|---|---|---|---|---|"]
    for n, c, a, mn, mx in sorted(rows, key=lambda r: -r[1] * r[2]):
        out.append(f"| `{n}` | {c} | {a:.0f} | {mn:.0f} | {mx:.0f} |")
    how = "by the call spans below" if span_line else "by the averages above"
    out += ["", f"One call = {call_name}: {call_ns:.0f} ns {how}.", work_line]
    out += ([span_line, ""] if span_line else [""])
    path = os.path.join(ROOT, "profiles", f"{name}_kernel_stats.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def bwd_call_spans(trace_dir):
    """Per backward call in a ``--kernel-trace`` run: the time from the start
    of its bwd_prep kernel to the end of the last bwd_* kernel dispatched
    before the next call's prep (ns)."""
    import csv
    import glob

    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return []
    ev = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            if "sdpa::dev::bwd_" in r["Kernel_Name"]:
                ev.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), "bwd_prep_kernel" in r["Kernel_Name"]))
    ev.sort()
    spans, start, end = [], None, None
    for t0, t1, is_prep in ev:
        if is_prep:
            if start is not None:
                spans.append(end - start)
            start, end = t0, t1
        elif start is not None:
            end = max(end, t1)
    if start is not None:
        spans.append(end - start)
    return spans


# SQ counters of the counter summaries, and what they show.
COUNTER_NOTES = {
    "SQ_WAVES": "waves launched",
    "SQ_INSTS_VALU": "vector ALU instructions (MFMA included)",
    "SQ_INSTS_MFMA": "MFMA instructions",
    "SQ_INSTS_LDS": "LDS instructions",
    "SQ_INSTS_SALU": "scalar ALU instructions",
    "SQ_INSTS_VALU_TRANS_F32": "transcendental float32 instructions (v_exp_f32 ...)",
    "SQ_VALU_MFMA_BUSY_CYCLES": "cycles the matrix cores are busy, summed over SIMDs",
    "SQ_BUSY_CYCLES": "cycles the SQs are busy",
    "SQ_WAVE_CYCLES": "wave-resident cycles (quad-cycle units)",
    "SQ_WAIT_ANY": "wave cycles waiting for anything: counters, barriers, dependencies (quad-cycles)",
    "SQ_WAIT_INST_ANY": "wave cycles waiting for any instruction's dependencies (quad-cycles)",
    "SQ_ACTIVE_INST_VALU": "wave cycles issuing VALU (quad-cycles)",
    "SQ_ACTIVE_INST_LDS": "wave cycles issuing LDS (quad-cycles)",
    "SQ_WAIT_INST_LDS": "wave cycles waiting on LDS (quad-cycles)",
    "SQ_LDS_BANK_CONFLICT": "LDS bank-conflict cycles",
    "SQ_INSTS_LDS_LOAD_BANDWIDTH": "LDS read bandwidth (64-byte units)",
    "GRBM_GUI_ACTIVE": "GPU busy cycles (summed over the 8 XCDs)",
}


def summarize_counters(dirs, name, commands, kernel_us):
    """Reduce ``rocprofv3 --pmc ... --output-format csv`` runs of ``bench.py
    --workload NAME`` to profiles/NAME_counters.md: each counter averaged over
    the attention dispatches, per-wave instruction counts, and the matrix
    cores' busy fraction of the elapsed cycles."""
    import csv
    import glob

    vals = {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if "attn_fwd_kernel" not in r["Kernel_Name"]:
                        continue
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    waves = avg.get("SQ_WAVES", 1.0)
    out = [f"# SQ counters: {name} (attention kernel)", "", "Commands (from /tmp with TMPDIR=/tmp; `$R` is the repository root):", ""]
    out += ["    " + c for c in commands]
    out += ["", "| counter | per dispatch | per wave | meaning |", "|---|---|---|---|"]
    for k in sorted(avg):
        out.append(f"| {k} | {avg[k]:,.0f} | {avg[k] / waves:,.1f} | {COUNTER_NOTES.get(k, '')} |")
    out.append("")
    if "SQ_INSTS_MFMA" in avg and "SQ_INSTS_VALU" in avg:
        out.append(f"VALU instructions per MFMA: {(avg['SQ_INSTS_VALU'] - avg['SQ_INSTS_MFMA']) / avg['SQ_INSTS_MFMA']:.2f}"
                   " (MFMA itself counts as VALU, so it is taken out).")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and "GRBM_GUI_ACTIVE" in avg:
        clk = avg["GRBM_GUI_ACTIVE"] / 8  # per XCD
        simd = 256 * 4
        busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / simd / clk
        out.append(f"Matrix cores busy: {100 * busy:.1f}% of the elapsed cycles per SIMD "
                   f"({clk:,.0f} busy cycles per XCD per dispatch under the counters; the bench times "
                   f"{kernel_us:.1f} us per call without them).")
    for a, b, what in (("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES", "issuing VALU"),
                       ("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES", "waiting on dependencies"),
                       ("SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "waiting on LDS")):
        if a in avg and b in avg and avg[b]:
            out.append(f"Share of wave cycles {what}: {100 * avg[a] / avg[b]:.1f}%.")
    out.append("")
    path = os.path.join(ROOT, "profiles", f"{name}_counters.md")
    with open(path, "w") as f:
        f.write("\n".join(out))
    print("\n".join(out))


def measure(s, steps, warmup, warm=False, event_every=EVENT_EVERY):
    """Time one workload.  HBM-bound workloads rotate over K/V copies that
    together exceed three times the Infinity Cache, so every step streams from
    HBM (cold, the graded number); ``warm`` keeps one copy, which the caches
    hold from one step to the next (context only)."""
    import torch

    floor = 3 * INFINITY_CACHE if bound(s) == "hbm" and not warm else 0
    r = BwdRunner(s) if s.get("bwd") else Runner(s, floor)
    ms, kms = time_steps(r, steps, warmup, event_every=event_every)
    flops, nbytes = work(s)
    kmean = sum(kms) / len(kms)
    kms_sorted = sorted(kms)
    res = dict(s)
    res.update(plan=r.plan, kv_sets=r.nsets, ms_per_step=ms, kernel_ms_mean=kmean, kernel_samples=len(kms),
               kernel_ms_p10=kms_sorted[len(kms) // 10], kernel_ms_p50=kms_sorted[len(kms) // 2],
               kernel_ms_p90=kms_sorted[(9 * len(kms)) // 10], flops=flops, bytes=nbytes, bound=bound(s))
    if res["bound"] == "hbm":
        res["achieved"] = nbytes / (kmean * 1e-3) / 1e9
        res["peak"] = HBM_PEAK_GBS
        res["unit"] = "GB/s"
        res["step_value"] = nbytes / (ms * 1e-3) / 1e9
    else:
        res["achieved"] = flops / (kmean * 1e-3) / 1e12
        res["peak"] = FP32_PEAK_TFLOPS if s["dtype"] == "f32" else MFMA16_PEAK_TFLOPS
        res["unit"] = "TFLOP/s"
        res["step_value"] = flops / (ms * 1e-3) / 1e12
    res["frac"] = res["achieved"] / res["peak"]
    torch.cuda.synchronize()
    return res, r


# The prefill half of the metric: the long causal D=256 layer (L = 32768,
# 16 query / 2 KV heads), then the other prefill workloads in brief (the
# encoder and vision layers, the windowed D=256 layers).
PREFILL = "causal_l32768_d256"
PREFILL_CONFIGS = ("encoder_h20_l1500_d64", "vision_h16_l1024_d72", "vision_h16_l4096_d72",
                   "window_l2048_d256", "window_l4096_d256", "window_l8192_d256")


def roofline_of(res, name):
    """The roofline object of a measured workload: algorithmic work per call
    over the call's device time (attention kernel plus the split combine)."""
    return {"bound": res["bound"], "achieved": round(res["achieved"], 3), "peak": res["peak"],
            "unit": res["unit"], "frac": round(res["frac"], 4), "traffic": traffic_from_profiles(name),
            "kernels": "attention + combine" if "splits=1 " not in res["plan"] else "attention",
            "kernel_us_mean": round(res["kernel_ms_mean"] * 1e3, 3),
            "kernel_us_median": round(res["kernel_ms_p50"] * 1e3, 3),
            "kernel_us_p10": round(res["kernel_ms_p10"] * 1e3, 3),
            "kernel_us_p90": round(res["kernel_ms_p90"] * 1e3, 3),
            "kernel_samples": res["kernel_samples"]}


def shape_config(s, res):
    return {"workload": s["name"], "B": s["b"], "Hq": s["hq"], "Hkv": s["hkv"], "Lq": s["lq"], "Lk": s["lk"],
            "Dqk": s["dqk"], "Dv": s["dv"], "mask": s["mask"], "window": s["window"],
            "mask_array": s["arr"], "kv_lens": kv_lengths(s) if s.get("varlen") else None,
            "pass": "backward" if s.get("bwd") else "forward", "kv_sets": res["kv_sets"], "plan": res["plan"]}


def prefill_report(steps, warmup, cpu):
    """The prefill half of the line: the long causal layer timed like the
    headline workload, then each other prefill workload with 10 warm-up and 40
    timed calls, every call sampled."""
    import torch

    s = SHAPES[PREFILL]
    print(f"prefill {PREFILL}", file=sys.stderr, flush=True)
    res, run = measure(s, steps, warmup)
    out = {"workload": PREFILL, "metric": "prefill TFLOP/s", "value": round(res["step_value"], 3),
           "unit": res["unit"], "ms_per_step": round(res["ms_per_step"], 5), "dtype": s["dtype"],
           "config": shape_config(s, res), "roofline": roofline_of(res, PREFILL),
           "cpu_baseline": cpu_baseline(s, run) if cpu else None}
    del run
    torch.cuda.empty_cache()
    rows = []
    for name in PREFILL_CONFIGS:
        sh = SHAPES[name]
        print(f"prefill {name}", file=sys.stderr, flush=True)
        r, run = measure(sh, MIN_SAMPLES, 10, event_every=1)
        rows.append({"workload": name, "plan": r["plan"],
                     "kernel_us_median": round(r["kernel_ms_p50"] * 1e3, 3),
                     "kernel_us_p10": round(r["kernel_ms_p10"] * 1e3, 3),
                     "kernel_us_p90": round(r["kernel_ms_p90"] * 1e3, 3),
                     "kernel_samples": r["kernel_samples"],
                     "tflops": round(r["flops"] / (r["kernel_ms_p50"] * 1e-3) / 1e12, 3),
                     "frac": round(r["flops"] / (r["kernel_ms_p50"] * 1e-3) / 1e12 / r["peak"], 4),
                     "cpu_baseline": cpu_baseline(sh, run, budget_s=4.0) if cpu else None})
        del run
        torch.cuda.empty_cache()
    out["configs"] = rows
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=160)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the default workload: leave out the prefill half of the line")
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(SHAPES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true", help="also time every shape of the table")
    ap.add_argument("--sweep-out", default="", help="with --sweep: also write the rows to this JSON file")
    ap.add_argument("--sweep-only", default="", help="comma-separated name prefixes to sweep")
    ap.add_argument("--warm", action="store_true",
                    help="with --sweep: time HBM-bound shapes on one resident K/V copy (cache-warm context)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: reduce FETCH_SIZE / WRITE_SIZE counter runs of --workload "
                         "into profiles/traffic_<workload>.json")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="with --summarize-pmc / --summarize-counters: the profiling commands, recorded in the summary")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="host only: reduce a rocprofv3 kernel-trace stats run of --workload into "
                         "profiles/<workload>_kernel_stats.md (--pmc-command gives the command)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="host only: reduce rocprofv3 SQ counter runs of --workload into profiles/<workload>_counters.md")
    ap.add_argument("--kernel-us", type=float, default=0.0,
                    help="with --summarize-counters: the bench's device time per call, for the clock estimate")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.workload, " ".join(args.pmc_command))
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload, args.pmc_command, args.kernel_us)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload,
                      args.calibrate_copy_mib, args.pmc_command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (got --gpus {args.gpus}): multi-GPU runs are not supported",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import scaled_dot_product_fwd_amd as sdpa

    sdpa.load()
    s = SHAPES[args.workload]
    res, runner = measure(s, args.steps, args.warmup)
    if args.calibrate_copy_mib:
        calibration_copy(args.calibrate_copy_mib)
    cpu = None if args.no_cpu_baseline else cpu_baseline(s, runner)
    vs = None
    if pages_shape(s):
        pages_us = PAGES_DECODE_US[(s["hkv"], s["lk"])]
        vs = res["step_value"] / (res["bytes"] / (pages_us * 1e-6) / 1e9)
    line = {
        "metric": METRIC,
        "value": round(res["step_value"], 3),
        "unit": res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None if vs is None else round(vs, 3),
        "dtype": s["dtype"],
        "data": "synthetic",
        "config": shape_config(s, res),
        "roofline": roofline_of(res, s["name"]),
        "cpu_baseline": cpu,
    }
    if args.workload == DEFAULT and not args.no_prefill:
        line["prefill"] = prefill_report(args.steps, args.warmup, not args.no_cpu_baseline)
    if args.workload == DEFAULT:
        line["context"] = context_rates()
    if args.sweep:
        rows = []
        prefixes = [p for p in args.sweep_only.split(",") if p]
        for sh in all_shapes():
            if prefixes and not any(sh["name"].startswith(p) for p in prefixes):
                continue
            print(f"sweep {sh['name']}", file=sys.stderr, flush=True)
            r, rr = measure(sh, MIN_SAMPLES, 10, warm=args.warm, event_every=1)
            del rr
            torch.cuda.empty_cache()
            rows.append({k: r[k] for k in ("name", "plan", "kv_sets", "ms_per_step", "kernel_ms_mean",
                                           "kernel_ms_p10", "kernel_ms_p50", "kernel_ms_p90", "flops",
                                           "bytes", "bound", "achieved", "peak", "unit", "frac",
                                           "step_value")})
            print(f"  {sh['name']:28s} kernel {r['kernel_ms_mean'] * 1e3:9.2f} us  step {r['ms_per_step'] * 1e3:9.2f} us"
                  f"  {r['achieved']:9.2f} {r['unit']:8s} {100 * r['frac']:6.2f}% of {r['bound']}",
                  file=sys.stderr, flush=True)
        if args.sweep_out:
            os.makedirs(os.path.dirname(args.sweep_out) or ".", exist_ok=True)
            with open(args.sweep_out, "w") as f:
                json.dump(rows, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
