"""Metamorphic checks on the GPU path (no oracle needed; they hold at any size).

* W2 = 0 or W1 = 0 gives Y = 0 exactly (SiLU(0) = 0);
* scaling W2 by 2^k scales Y by 2^k bit for bit (every partial sum of Up
  scales exactly; bf16 rounding commutes with powers of two in range);
* permuting rows of A permutes rows of Y; permuting Gate/Up column pairs
  permutes columns of Y (bitwise, full tiles);
* two runs give identical bits (no races between waves or workgroups).
"""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import Run, configs_of, dev, host, log

pytestmark = pytest.mark.gpu

SHAPE = (512, 512, 256)  # full tiles for every compiled tile size


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


@pytest.fixture(scope="module")
def data():
    M, N, K = SHAPE
    a, w1, w2 = I.make_inputs(M, K, N, 77)
    return a, w1, w2


def _run(handle, cfg, a, w1, w2):
    M, K = a.shape
    N = w1.shape[1]
    info = sw.swiglu_config_info(cfg)
    r = Run(handle)
    if info["variant"] == sw.VARIANT_INTERLEAVE:
        return host(r.fused(dev(a), dev(I.interleave_columns(w1, w2)), None, M, N, K,
                            sw.LAYOUT_INTERLEAVED, cfg, sw.VARIANT_INTERLEAVE))
    return host(r.fused(dev(a), dev(w1), dev(w2), M, N, K, sw.LAYOUT_SEPARATE, cfg,
                        sw.VARIANT_SYNC))


FUSED = configs_of(sw.VARIANT_INTERLEAVE) + configs_of(sw.VARIANT_SYNC)


@pytest.mark.parametrize("cfg", FUSED)
def test_zero_weight_gives_zero(handle, data, cfg):
    a, w1, w2 = data
    log(f"zero weights, config {cfg}")
    z = np.zeros_like(w1)
    for args in ((w1, z), (z, w2)):
        y = _run(handle, cfg, a, *args)
        assert np.all((y & 0x7FFF) == 0), "expected +-0 everywhere"


@pytest.mark.parametrize("cfg", FUSED)
def test_power_of_two_scaling_and_determinism(handle, data, cfg):
    a, w1, w2 = data
    log(f"scaling and determinism, config {cfg}")
    y = _run(handle, cfg, a, w1, w2)
    y2 = _run(handle, cfg, a, w1, w2)
    assert np.array_equal(y, y2), "two runs differ"
    k = 3
    w2s = I.f32_to_bf16_bits(I.bf16_bits_to_f32(w2) * np.float32(2.0 ** k))
    ys = _run(handle, cfg, a, w1, w2s)
    expect = I.f32_to_bf16_bits(I.bf16_bits_to_f32(y) * np.float32(2.0 ** k))
    assert np.array_equal(ys, expect)


@pytest.mark.parametrize("cfg", FUSED)
def test_permutation_equivariance(handle, data, cfg):
    a, w1, w2 = data
    log(f"permutations, config {cfg}")
    rng = np.random.default_rng(cfg)
    y = _run(handle, cfg, a, w1, w2)
    pr = rng.permutation(a.shape[0])
    pc = rng.permutation(w1.shape[1])
    yp = _run(handle, cfg, a[pr], w1[:, pc], w2[:, pc])
    assert np.array_equal(yp, y[pr][:, pc])
