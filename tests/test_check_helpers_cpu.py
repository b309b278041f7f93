"""The whole-output checkers the GPU tests use (gpu_util.full_check and
gpu_util.rounding_check), exercised on the CPU with planted mistakes: they
must pass exact results and fail each kind of error they exist to catch."""
import numpy as np
import pytest

import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import full_check, rounding_check


def _ref(shape=(300, 200), seed=0):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def test_full_check_passes_the_rounded_reference():
    y = _ref()
    s = full_check(oracle.round_bf16(y), y, "exact")
    assert s["elements"] == y.size and s["rel_gt_1pct"] == 0.0 and s["worst_frac"] < 0.5


@pytest.mark.parametrize("plant", ["two_percent", "nan", "sign", "absolute_floor"])
def test_full_check_catches_planted_errors(plant):
    y = _ref()
    bits = oracle.round_bf16(y)
    if plant == "two_percent":
        bits[123 // 200, 123 % 200] = oracle.round_bf16(np.float32(y[0, 123] * 1.02)[None])[0]
    elif plant == "nan":
        bits[299, 199] = 0xFFFF
    elif plant == "sign":
        bits[7, 3] ^= 0x8000
    else:  # a near-zero element off by more than the 2^-10 floor
        y[5, 5] = np.float32(1e-6)
        bits = oracle.round_bf16(y)
        bits[5, 5] = oracle.round_bf16(np.float32(3e-3)[None])[0]
    with pytest.raises(AssertionError):
        full_check(bits, y, plant)


def test_rounding_check_accepts_rne_and_order_flips():
    K = 1024
    g = _ref(seed=1)
    bits = oracle.round_bf16(g)
    assert rounding_check(bits, g, K, "rne") == 0
    # put one value a hair below a rounding midpoint: the neighbour above is
    # what a sum differing only in order may round to
    lo = I.bf16_bits_to_f32(np.array([0x3F80], np.uint16))[0]   # 1.0
    hi = I.bf16_bits_to_f32(np.array([0x3F81], np.uint16))[0]   # 1.0078125
    g[0, 0] = np.float32((lo + hi) / 2 - 1e-7)
    bits = oracle.round_bf16(g)
    assert bits[0, 0] == 0x3F80
    bits[0, 0] = 0x3F81
    assert rounding_check(bits, g, K, "flip") == 1


@pytest.mark.parametrize("plant", ["one_step_far_from_midpoint", "two_steps", "sign"])
def test_rounding_check_catches_planted_errors(plant):
    K = 1024
    g = _ref(seed=2)
    g[0, 0] = np.float32(1.25)  # exactly representable: far from any midpoint
    bits = oracle.round_bf16(g)
    if plant == "one_step_far_from_midpoint":
        bits[0, 0] += 1
    elif plant == "two_steps":
        bits[10, 10] += 2
    else:
        bits[20, 20] ^= 0x8000
    with pytest.raises(AssertionError):
        rounding_check(bits, g, K, plant)
