"""GPU parity at head dim 512 (and dims above 256, zero-padded to it) against
the float64 oracle: every query length runs the one 512 arrangement (two
32-row groups whose waves split the dv tiles), with the masks, mask arrays,
per-batch lengths and split plans of the other head dims.
"""

import zlib

import pytest
import torch

from gpu_cases import check_full, check_sampled
from scaled_dot_product_fwd_amd.synth import additive_mask, bool_mask

pytestmark = pytest.mark.gpu


def _say(*a):
    print("CASE", *a, flush=True)


CASES = [
    # b, hq, hkv, lq, lk, dqk, dv, dtype, mask, window
    (1, 4, 2, 150, 150, 512, 512, "bf16", "causal", 0),
    (1, 2, 2, 130, 333, 512, 512, "f16", "none", 0),
    (1, 16, 4, 1, 2000, 512, 512, "bf16", "causal", 0),
    (1, 32, 8, 8, 1500, 512, 512, "f16", "causal", 0),
    (2, 4, 2, 100, 260, 512, 512, "bf16", "window", 45),
    (1, 4, 4, 70, 70, 320, 320, "bf16", "none", 0),
    (1, 8, 2, 20, 400, 512, 384, "f16", "causal", 0),
    (1, 2, 1, 33, 97, 488, 512, "bf16", "none", 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) for x in c))
def test_d512_cases(case):
    b, hq, hkv, lq, lk, dqk, dv, dt, mask, w = case
    _say(case)
    check_full(b, hq, hkv, lq, lk, dqk, dv, dt, mask, w, seed=zlib.crc32(repr(case).encode()) % 10000)


@pytest.mark.parametrize("splits", [1, 5, 32])
def test_d512_forced_splits(splits):
    _say("d512 splits", splits)
    check_full(1, 8, 2, 2, 1200, 512, 512, "bf16", "none", 0, seed=splits, num_splits=splits)


@pytest.mark.parametrize("kind", ["bool", "add"])
def test_d512_mask_arrays(kind):
    _say("d512 mask array", kind)
    shape = (1, 4, 90, 200)
    arr = bool_mask(shape, 3, keep=0.7) if kind == "bool" else additive_mask(shape, 3, torch.bfloat16)
    check_full(1, 4, 2, 90, 200, 512, 512, "bf16", "causal", 0, seed=8, attn_mask=arr)


def test_d512_causal_prefill_sampled():
    """Full-size causal prefill L=4096, Hq=8, Hkv=2; sampled rows."""
    _say("d512 causal prefill L=4096")
    check_sampled(1, 8, 2, 4096, 4096, 512, 512, "bf16", "causal", 0, seed=51, nrows=24)


def test_d512_decode_sampled():
    """Decode Lq=1, Hq=32, Hkv=8, Lk=16384; sampled rows."""
    _say("d512 decode Lk=16384")
    check_sampled(1, 32, 8, 1, 16384, 512, 512, "bf16", "causal", 0, seed=52, nrows=32)
