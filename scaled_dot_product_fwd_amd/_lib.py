"""ctypes view of libsdpa_fwd.so: the C ABI of include/sdpa.h, same names.

Argument marshalling only; every step of the computation runs in the HIP
kernels behind ``sdpa_forward``.  A missing library is an error, never a
fallback.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa_fwd.so")

SDPA_F32, SDPA_F16, SDPA_BF16 = 0, 1, 2
SDPA_MASK_NONE, SDPA_MASK_CAUSAL, SDPA_MASK_WINDOW = 0, 1, 2
SDPA_MASK_ARRAY_NONE, SDPA_MASK_ARRAY_BOOL, SDPA_MASK_ARRAY_ADD = 0, 1, 2

STATUS = {
    0: "SDPA_OK",
    -1: "SDPA_E_NULL",
    -2: "SDPA_E_SHAPE",
    -3: "SDPA_E_HEAD_DIM",
    -4: "SDPA_E_DTYPE",
    -5: "SDPA_E_MASK",
    -6: "SDPA_E_STRIDE",
    -7: "SDPA_E_WORKSPACE",
    -8: "SDPA_E_SCALE",
    -9: "SDPA_E_DEVICE",
    -10: "SDPA_E_HIP",
    -11: "SDPA_E_PLAN",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

EXPORTED = ("sdpa_desc_init", "sdpa_workspace_bytes", "sdpa_forward", "sdpa_forward_masked",
            "sdpa_forward_varlen", "sdpa_forward_noalloc", "sdpa_backward_workspace_bytes", "sdpa_backward", "sdpa_backward_varlen",
            "sdpa_describe_plan",
            "sdpa_set_profile_events", "sdpa_last_error")


class sdpa_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads_q", ctypes.c_int64),
        ("heads_kv", ctypes.c_int64),
        ("len_q", ctypes.c_int64),
        ("len_k", ctypes.c_int64),
        ("dim_qk", ctypes.c_int64),
        ("dim_v", ctypes.c_int64),
        ("q_stride", ctypes.c_int64 * 3),
        ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3),
        ("o_stride", ctypes.c_int64 * 3),
        ("dtype", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("num_splits", ctypes.c_int32),
        ("row_tile", ctypes.c_int32),
        ("mask_array", ctypes.c_int32),
        ("mask_stride", ctypes.c_int64 * 3),
    ]


class SdpaError(Exception):
    """Base of the errors raised for a failed library call."""


class SdpaValueError(SdpaError, ValueError):
    """Validation failure: the message names the violated constraint."""


class SdpaRuntimeError(SdpaError, RuntimeError):
    """Device or HIP runtime failure."""


_lib = None


def load() -> ctypes.CDLL:
    """Load (once) and return the library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m scaled_dot_product_fwd_amd.build_lib`")
    try:
        # PyTorch ships its own HIP runtime (SONAME libamdhip64.so.7).  Loading
        # torch first makes the library bind to that same runtime instead of
        # bringing a second copy into the process.
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.sdpa_desc_init.argtypes = [P(sdpa_desc_t)] + [ctypes.c_int64] * 7 + [ctypes.c_int32]
    lib.sdpa_desc_init.restype = ctypes.c_int
    lib.sdpa_workspace_bytes.argtypes = [P(sdpa_desc_t), P(ctypes.c_size_t)]
    lib.sdpa_workspace_bytes.restype = ctypes.c_int
    lib.sdpa_forward.argtypes = [P(sdpa_desc_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                 ctypes.c_void_p]
    lib.sdpa_forward.restype = ctypes.c_int
    lib.sdpa_forward_masked.argtypes = [P(sdpa_desc_t), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
    lib.sdpa_forward_masked.restype = ctypes.c_int
    lib.sdpa_forward_varlen.argtypes = [P(sdpa_desc_t)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t,
                                                                                    ctypes.c_void_p]
    lib.sdpa_forward_varlen.restype = ctypes.c_int
    lib.sdpa_forward_noalloc.argtypes = [P(sdpa_desc_t)] + [ctypes.c_void_p] * 9
    lib.sdpa_forward_noalloc.restype = ctypes.c_int
    lib.sdpa_backward_workspace_bytes.argtypes = [P(sdpa_desc_t), P(ctypes.c_size_t)]
    lib.sdpa_backward_workspace_bytes.restype = ctypes.c_int
    lib.sdpa_backward.argtypes = [P(sdpa_desc_t)] + [ctypes.c_void_p] * 10 + [ctypes.c_size_t, ctypes.c_void_p]
    lib.sdpa_backward.restype = ctypes.c_int
    lib.sdpa_backward_varlen.argtypes = [P(sdpa_desc_t)] + [ctypes.c_void_p] * 13 + [ctypes.c_size_t,
                                                                                     ctypes.c_void_p]
    lib.sdpa_backward_varlen.restype = ctypes.c_int
    lib.sdpa_describe_plan.argtypes = [P(sdpa_desc_t), ctypes.c_char_p, ctypes.c_size_t]
    lib.sdpa_describe_plan.restype = ctypes.c_int
    lib.sdpa_set_profile_events.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    lib.sdpa_set_profile_events.restype = ctypes.c_int
    lib.sdpa_last_error.argtypes = []
    lib.sdpa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def sdpa_last_error() -> str:
    return load().sdpa_last_error().decode()


def check(rc: int) -> None:
    """Raise the Python error matching a non-zero status."""
    if rc == 0:
        return
    msg = f"{STATUS.get(rc, rc)}: {sdpa_last_error()}"
    if rc in (-9, -10):
        raise SdpaRuntimeError(msg)
    err = SdpaValueError(msg)
    err.status = rc
    raise err


def sdpa_desc_init(batch, heads_q, heads_kv, len_q, len_k, dim_qk, dim_v, dtype) -> sdpa_desc_t:
    d = sdpa_desc_t()
    check(load().sdpa_desc_init(ctypes.byref(d), batch, heads_q, heads_kv, len_q, len_k, dim_qk,
                                dim_v, dtype))
    return d


def sdpa_workspace_bytes(desc: sdpa_desc_t) -> int:
    n = ctypes.c_size_t(0)
    check(load().sdpa_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def sdpa_describe_plan(desc: sdpa_desc_t) -> str:
    buf = ctypes.create_string_buffer(512)
    check(load().sdpa_describe_plan(ctypes.byref(desc), buf, len(buf)))
    return buf.value.decode()


def sdpa_set_profile_events(start: int | None, stop: int | None) -> None:
    """Record two hipEvent_t handles around the next call's attention kernel."""
    check(load().sdpa_set_profile_events(start or None, stop or None))


def sdpa_forward(desc: sdpa_desc_t, q: int, k: int, v: int, o: int, lse: int | None,
                 workspace: int | None, workspace_bytes: int, stream: int | None) -> None:
    """Raw call with integer device addresses; raises on a non-zero status."""
    check(load().sdpa_forward(ctypes.byref(desc), q, k, v, o, lse or None, workspace or None,
                              workspace_bytes, stream or None))


def sdpa_forward_masked(desc: sdpa_desc_t, q: int, k: int, v: int, mask: int | None, o: int,
                        lse: int | None, workspace: int | None, workspace_bytes: int,
                        stream: int | None) -> None:
    """Raw call with an explicit mask array; raises on a non-zero status."""
    check(load().sdpa_forward_masked(ctypes.byref(desc), q, k, v, mask or None, o, lse or None,
                                     workspace or None, workspace_bytes, stream or None))


def sdpa_forward_varlen(desc: sdpa_desc_t, q: int, k: int, v: int, mask: int | None,
                        q_lens: int | None, kv_lens: int | None, o: int, lse: int | None,
                        workspace: int | None, workspace_bytes: int, stream: int | None) -> None:
    """Raw call with per-batch lengths (device int32 arrays); raises on a non-zero status."""
    check(load().sdpa_forward_varlen(ctypes.byref(desc), q, k, v, mask or None, q_lens or None,
                                     kv_lens or None, o, lse or None, workspace or None,
                                     workspace_bytes, stream or None))


def sdpa_forward_noalloc(desc: sdpa_desc_t, q: int, k: int, v: int, mask: int | None,
                         q_lens: int | None, kv_lens: int | None, o: int, lse: int | None,
                         stream: int | None) -> None:
    """Raw call of the forward that allocates nothing (split partials in the
    library's fixed per-device scratch); raises on a non-zero status."""
    check(load().sdpa_forward_noalloc(ctypes.byref(desc), q, k, v, mask or None, q_lens or None,
                                      kv_lens or None, o, lse or None, stream or None))


def sdpa_backward_workspace_bytes(desc: sdpa_desc_t) -> int:
    n = ctypes.c_size_t(0)
    check(load().sdpa_backward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)))
    return int(n.value)


def sdpa_backward(desc: sdpa_desc_t, q: int, k: int, v: int, o: int, dout: int, lse: int, dq: int, dk: int,
                  dv: int, workspace: int | None, workspace_bytes: int, stream: int | None) -> None:
    """Raw backward call with integer device addresses; raises on a non-zero status."""
    check(load().sdpa_backward(ctypes.byref(desc), q, k, v, o, dout, lse, dq, dk, dv, workspace or None,
                               workspace_bytes, stream or None))


def sdpa_backward_varlen(desc: sdpa_desc_t, q: int, k: int, v: int, mask: int, q_lens: int, kv_lens: int, o: int,
                         dout: int, lse: int, dq: int, dk: int, dv: int, workspace: int | None,
                         workspace_bytes: int, stream: int | None) -> None:
    """Raw backward call with a mask array and / or per-batch lengths (0 for an
    absent one); raises on a non-zero status."""
    check(load().sdpa_backward_varlen(ctypes.byref(desc), q, k, v, mask or None, q_lens or None, kv_lens or None,
                                      o, dout, lse, dq, dk, dv, workspace or None, workspace_bytes,
                                      stream or None))
