"""GPU parity at the full sizes of the five benchmark workloads.

The HIP path runs each workload at its real shape in the launch configuration
the bench times; the oracle recomputes sampled rows one by one (first and last
rows, window edges and random rows; 256 per shape, every row of the decode
shapes and of speculative verify up to Lq = 8) from the same seeded inputs.
The NaN-filled outputs show that every element was written.  Seeds follow
1000 * workload + shape index.
"""

import pytest

from gpu_cases import check_full, check_sampled

pytestmark = pytest.mark.gpu


def _say(*a):
    print("CASE", *a, flush=True)


def test_tiny_noncausal_fp32():
    _say("tiny fp32 B1 H4 L128 D64")
    check_full(1, 4, 4, 128, 128, 64, 64, "f32", "none", 0, seed=1000)


DECODE_LK = [256, 1024, 4096, 8192, 16384, 32768]


@pytest.mark.parametrize("hkv", [4, 8])
@pytest.mark.parametrize("lk", DECODE_LK)
def test_decode_gqa_asymmetric(hkv, lk):
    _say("decode", hkv, lk)
    idx = DECODE_LK.index(lk) + (0 if hkv == 4 else len(DECODE_LK))
    check_sampled(1, 64, hkv, 1, lk, 192, 128, "bf16", "causal", 0, seed=2000 + idx, nrows=64)


VERIFY_LQ = [1, 2, 4, 8, 12, 16, 24, 32, 48, 64]


@pytest.mark.parametrize("lk", [16384, 32768])
@pytest.mark.parametrize("lq", VERIFY_LQ)
def test_speculative_verify(lk, lq):
    _say("verify", lk, lq)
    idx = VERIFY_LQ.index(lq) + (0 if lk == 16384 else len(VERIFY_LQ))
    check_sampled(1, 32, 8, lq, lk, 128, 128, "f16", "none", 0, seed=3000 + idx, nrows=256)


def test_encoder_prefill_d64():
    _say("encoder H20 L1500 D64")
    check_sampled(1, 20, 20, 1500, 1500, 64, 64, "bf16", "none", 0, seed=4000, nrows=256)


@pytest.mark.parametrize("L", [1024, 4096])
def test_vision_prefill_d72(L):
    _say("vision H16 D72", L)
    check_sampled(1, 16, 16, L, L, 72, 72, "bf16", "none", 0, seed=4001 + (L == 4096), nrows=256)


@pytest.mark.parametrize("L", [2048, 4096, 8192])
def test_window_prefill_d256(L):
    _say("window prefill D256", L)
    idx = [2048, 4096, 8192].index(L)
    check_sampled(1, 16, 8, L, L, 256, 256, "bf16", "window", 1024, seed=5000 + idx, nrows=256)


def test_full_causal_32k_d256():
    _say("causal 32k D256")
    check_sampled(1, 16, 2, 32768, 32768, 256, 256, "bf16", "causal", 0, seed=5003, nrows=256)
