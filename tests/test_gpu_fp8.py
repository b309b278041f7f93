"""GPU parity of the FP8 (OCP E4M3) path against the CPU oracle.

* quantisation: every bf16 bit pattern, several scales, bit for bit;
* the k-major Gate/Up pack: bit for bit;
* the forward, in both kernel orders (interleave and sync, on the same W8):
  every FP8 configuration on seeded shapes with ragged tails in M, N and K,
  launches that exercise the split tail, K = 0, and the five Qwen2.5-shaped
  workloads at full size in the table's configuration, every element of Y
  against the oracle's full Y.  Bar: |y - y_ref| <= 0.01 |y_ref| + 2^-10 against the oracle's
  fp32 value computed from the same E4M3 codes and scales.

Input recipe: the seeded bf16 draws of the bf16 tests (A ~ N(0, 1),
W ~ N(0, 1/K)), quantised by the oracle with one scale per tensor,
scale = max|x| / 448 (the tensor's largest magnitude maps to the largest
E4M3 value).
"""
import time

import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import assert_parity, decode, empty_poisoned, full_check, host, log

pytestmark = pytest.mark.gpu


def torch():
    import torch as t
    return t


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


def dev8(codes):
    return torch().from_numpy(np.ascontiguousarray(codes)).cuda()


def host8(t):
    return t.cpu().numpy()


def quantised(x):
    """(codes, scale) of an fp32 array: scale = max|x| / 448 in fp32."""
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(1.0)
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    return oracle.quantize_e4m3(x, np.float32(1.0) / s), float(s)


def fp8_inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((M, K), dtype=np.float32)
    s = np.float32(1.0 / np.sqrt(max(K, 1)))
    w1 = rng.standard_normal((K, N), dtype=np.float32) * s
    w2 = rng.standard_normal((K, N), dtype=np.float32) * s
    (a8, sa), (w18, s1), (w28, s2) = quantised(a), quantised(w1), quantised(w2)
    return a8, w18, w28, sa, s1, s2


def variant_of(cfg):
    v = sw.swiglu_config_info(cfg)["variant"]
    return {sw.VARIANT_FP8_SYNC: sw.VARIANT_SYNC,
            sw.VARIANT_FP8_PACKED: sw.VARIANT_FP8_PACKED}.get(v, sw.VARIANT_INTERLEAVE)


def forward(handle, a8, w8, M, N, K, scales, cfg=-1, variant=sw.VARIANT_AUTO):
    t = torch()
    y = empty_poisoned((M, N))
    if cfg >= 0:
        variant = variant_of(cfg)
    sw.swiglu_forward_fp8(handle, dev8(a8), dev8(w8), y, M, N, K, *scales, config_id=cfg,
                          variant=variant)
    t.cuda.synchronize()
    return host(y)


# --------------------------------------------------------------------------- quantise
@pytest.mark.parametrize("inv_scale", [1.0, 64.0, 0.001953125, 3.0, 81.37])
def test_quantize_every_bf16_pattern(handle, inv_scale):
    t = torch()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = t.from_numpy(bits.view(np.int16)).cuda()
    q = t.full((65536,), 0x55, dtype=t.uint8, device="cuda")
    sw.swiglu_quantize_fp8(handle, x, q, 65536, inv_scale)
    t.cuda.synchronize()
    got = host8(q)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = oracle.quantize_e4m3(I.bf16_bits_to_f32(bits), inv_scale)
    nan_in = np.isnan(I.bf16_bits_to_f32(bits))
    # NaN inputs: the NaN code of either sign (the sign of a NaN product is not fixed)
    assert np.all((got[nan_in] & 0x7F) == 0x7F)
    assert np.array_equal(got[~nan_in], ref[~nan_in])


def test_quantize_rejects_bad_arguments(handle):
    t = torch()
    x = t.zeros(32, dtype=t.int16, device="cuda")
    q = t.zeros(32, dtype=t.uint8, device="cuda")
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_quantize_fp8(handle, x, q, 24)            # not a multiple of 16
    assert e.value.status == sw.ERR_UNSUPPORTED
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_quantize_fp8(handle, x, x, 32)            # output overlaps input
    assert e.value.status == sw.ERR_INVALID_ARG


# --------------------------------------------------------------------------- pack
@pytest.mark.parametrize("K,N", [(16, 8), (208, 264), (896, 4864), (1536, 8960)])
def test_pack_fp8_bitwise(handle, K, N):
    t = torch()
    rng = np.random.default_rng(K + N)
    w1 = rng.integers(0, 256, (K, N), dtype=np.uint8)
    w2 = rng.integers(0, 256, (K, N), dtype=np.uint8)
    w8 = t.full((2 * N, K), 0x55, dtype=t.uint8, device="cuda")
    sw.swiglu_pack_fp8(handle, dev8(w1), dev8(w2), w8, K, N)
    t.cuda.synchronize()
    assert np.array_equal(host8(w8), oracle.pack_fp8_kmajor(w1, w2))


# --------------------------------------------------------------------------- forward
SHAPES = [
    (300, 264, 208),   # 2 x 256-row tiles (ragged), ragged column tiles, K tail of 16
    (37, 136, 528),    # ragged 64-row tiles, long K
    (1, 8, 16),        # one row, one 8-column chunk, one 16-byte k run
    (129, 520, 96),    # one row past a tile, K = 1.5 steps
]


def fp8_configs():
    return [i for i in range(sw.swiglu_config_count())
            if sw.swiglu_config_info(i)["variant"] in (sw.VARIANT_FP8, sw.VARIANT_FP8_SYNC)]


@pytest.fixture(scope="module")
def cases():
    out = {}
    for i, (M, N, K) in enumerate(SHAPES):
        a8, w18, w28, sa, s1, s2 = fp8_inputs(M, N, K, 300 + i)
        y = oracle.swiglu_fp8_rows(a8, w18, w28, sa, s1, s2)
        out[(M, N, K)] = dict(a8=a8, w8=oracle.pack_fp8_kmajor(w18, w28), s=(sa, s1, s2), y=y)
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", fp8_configs())
def test_fp8_config_parity(handle, cases, cfg, shape):
    M, N, K = shape
    c = cases[shape]
    log(f"fp8 config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y = forward(handle, c["a8"], c["w8"], M, N, K, c["s"], cfg)
    assert_parity(y, c["y"], f"fp8 cfg {cfg} {shape}")


@pytest.mark.parametrize("cfg", [i for i in fp8_configs()
                                 if sw.swiglu_config_info(i)["tail_split"]])
def test_fp8_split_tail_parity(handle, cfg):
    """Whole rounds of big tiles plus a short last round run as quarter tiles."""
    info = sw.swiglu_config_info(cfg)
    cus = torch().cuda.get_device_properties(0).multi_processor_count
    bm, bn = info["bm"], info["bn"]
    M = 8 * bm - 40
    ntn = cus // 8 + 1
    N = ntn * bn - 8
    K = 80
    nt = 8 * ntn
    assert nt // cus > 0 and 0 < 4 * (nt % cus) <= cus
    a8, w18, w28, sa, s1, s2 = fp8_inputs(M, N, K, 901)
    log(f"fp8 split-tail config {cfg} shape {(M, N, K)}")
    y = forward(handle, a8, oracle.pack_fp8_kmajor(w18, w28), M, N, K, (sa, s1, s2), cfg)
    assert_parity(y, oracle.swiglu_fp8_rows(a8, w18, w28, sa, s1, s2), f"fp8 split cfg {cfg}")


def test_fp8_k_zero_and_errors(handle):
    t = torch()
    M, N = 40, 72
    y = t.full((M, N), -1, dtype=t.int16, device="cuda")
    sw.swiglu_forward_fp8(handle, 0, 0, y, M, N, 0)
    t.cuda.synchronize()
    assert np.all(decode(host(y)) == 0.0)
    a = t.zeros((M, 24), dtype=t.uint8, device="cuda")
    w = t.zeros((2 * N, 24), dtype=t.uint8, device="cuda")
    with pytest.raises(sw.SwiGLUError) as e:               # K % 16 != 0
        sw.swiglu_forward_fp8(handle, a, w, y, M, N, 24)
    assert e.value.status == sw.ERR_UNSUPPORTED
    with pytest.raises(sw.SwiGLUError) as e:               # a bf16 config id
        sw.swiglu_forward_fp8(handle, a, w, y, M, N, 16, config_id=0)
    assert e.value.status == sw.ERR_INVALID_ARG
    sync_cfg = [i for i in fp8_configs() if variant_of(i) == sw.VARIANT_SYNC][0]
    with pytest.raises(sw.SwiGLUError) as e:               # a sync config, interleave order
        sw.swiglu_forward_fp8(handle, a, w, y, M, N, 16, config_id=sync_cfg,
                              variant=sw.VARIANT_INTERLEAVE)
    assert e.value.status == sw.ERR_INVALID_ARG
    with pytest.raises(sw.SwiGLUError) as e:               # not an FP8 order
        sw.swiglu_forward_fp8(handle, a, w, y, M, N, 16, variant=sw.VARIANT_GEMM)
    assert e.value.status == sw.ERR_INVALID_ARG
    y.fill_(-1)                                            # K = 0 in sync order
    sw.swiglu_forward_fp8(handle, 0, 0, y, M, N, 0, variant=sw.VARIANT_SYNC)
    t.cuda.synchronize()
    assert np.all(decode(host(y)) == 0.0)


def test_fp8_scales_apply_before_silu(handle):
    """Scaling s_w2 by 2^k scales Y by 2^k (Up is linear); halving s_w1
    changes Y non-linearly, as the oracle says."""
    M, N, K = 64, 128, 256
    a8, w18, w28, sa, s1, s2 = fp8_inputs(M, N, K, 77)
    w8 = oracle.pack_fp8_kmajor(w18, w28)
    for variant in (sw.VARIANT_INTERLEAVE, sw.VARIANT_SYNC):
        for scales in [(sa, s1, s2), (sa, s1, s2 * 8), (sa, s1 * 0.5, s2), (sa * 4, s1, s2)]:
            y = forward(handle, a8, w8, M, N, K, scales, variant=variant)
            assert_parity(y, oracle.swiglu_fp8_rows(a8, w18, w28, *scales),
                          f"fp8 variant {variant} scales {scales}")


# --------------------------------------------------------------------------- workloads
@pytest.fixture(scope="module", params=I.WORKLOADS, ids=lambda w: w.name)
def workload(request):
    w = request.param
    log(f"fp8 inputs for {w.name} M={w.M} K={w.K} N={w.N}")
    a, w1, w2 = I.workload_inputs(w)
    (a8, sa), (w18, s1), (w28, s2) = (quantised(I.bf16_bits_to_f32(x)) for x in (a, w1, w2))
    del a, w1, w2
    t0 = time.perf_counter()
    y_ref = oracle.swiglu_fp8_rows(a8, w18, w28, sa, s1, s2)
    log(f"fp8 {w.name}: oracle full Y in {time.perf_counter() - t0:.1f} s")
    w8 = oracle.pack_fp8_kmajor(w18, w28)
    return dict(w=w, a8=a8, w8=w8, p8=oracle.pack_fp8_fragments(w8), w18=w18, w28=w28,
                s=(sa, s1, s2), y_ref=y_ref)


@pytest.mark.parametrize("variant", [sw.VARIANT_AUTO, sw.VARIANT_SYNC, sw.VARIANT_FP8_PACKED],
                         ids=["auto", "sync", "packed"])
def test_fp8_workload_parity(handle, workload, variant):
    """Every output element of the FP8 forward at full size, in both kernel
    orders and on fragment-ordered weights."""
    d = workload
    w = d["w"]
    cfg = sw.swiglu_query_fp8(handle, w.M, w.N, w.K, variant)
    log(f"fp8 {w.name} variant {variant}: config {cfg['id']}")
    wt = d["p8"] if variant == sw.VARIANT_FP8_PACKED else d["w8"]
    y = forward(handle, d["a8"], wt, w.M, w.N, w.K, d["s"], variant=variant)
    s = full_check(y, d["y_ref"], f"fp8 {w.name} variant {variant}")
    log(f"fp8 {w.name} variant {variant}: all {s['elements']} elements within the bar "
        f"(worst {s['worst_frac']:.3f}); share > 1 % off: {s['rel_gt_1pct']:.2e}")


def test_fp8_workload_device_pack_and_quantise_match(handle, workload):
    """At full size the device pack reproduces the oracle's W8, and the device
    quantiser reproduces the oracle's codes of A."""
    t = torch()
    d = workload
    w = d["w"]
    w8 = t.empty((2 * w.N, w.K), dtype=t.uint8, device="cuda")
    sw.swiglu_pack_fp8(handle, dev8(d["w18"]), dev8(d["w28"]), w8, w.K, w.N)
    t.cuda.synchronize()
    assert np.array_equal(host8(w8), d["w8"])
    p8 = t.full((sw.swiglu_fp8_packed_bytes(w.N, w.K),), 0x55, dtype=t.uint8, device="cuda")
    sw.swiglu_pack_fp8_fragments(handle, w8, p8, w.K, w.N)
    t.cuda.synchronize()
    assert np.array_equal(host8(p8), d["p8"])
    del w8, p8
    a = I.make_a(w.M, w.K, 1000 * w.index + I.TENSOR_A)
    xa = t.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    q = t.empty((w.M, w.K), dtype=t.uint8, device="cuda")
    sw.swiglu_quantize_fp8(handle, xa, q, w.M * w.K, float(np.float32(1.0) / np.float32(d["s"][0])))
    t.cuda.synchronize()
    assert np.array_equal(host8(q), d["a8"])


# --------------------------------------------------------------------------- fragment order
def fp8_packed_configs():
    return [i for i in range(sw.swiglu_config_count())
            if sw.swiglu_config_info(i)["variant"] == sw.VARIANT_FP8_PACKED]


PACKED_SHAPES = SHAPES + [(33, 72, 144), (16, 4864, 896)]


@pytest.fixture(scope="module")
def packed_cases():
    out = {}
    for i, (M, N, K) in enumerate(PACKED_SHAPES):
        a8, w18, w28, sa, s1, s2 = fp8_inputs(M, N, K, 500 + i)
        w8 = oracle.pack_fp8_kmajor(w18, w28)
        out[(M, N, K)] = dict(a8=a8, w8=w8, p8=oracle.pack_fp8_fragments(w8), s=(sa, s1, s2),
                              y=oracle.swiglu_fp8_rows(a8, w18, w28, sa, s1, s2))
    return out


@pytest.mark.parametrize("shape", PACKED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fp8_fragment_pack_bitwise(handle, packed_cases, shape):
    t = torch()
    M, N, K = shape
    c = packed_cases[shape]
    p8 = t.full((sw.swiglu_fp8_packed_bytes(N, K),), 0x55, dtype=t.uint8, device="cuda")
    sw.swiglu_pack_fp8_fragments(handle, dev8(c["w8"]), p8, K, N)
    t.cuda.synchronize()
    assert np.array_equal(host8(p8), c["p8"])


@pytest.mark.parametrize("shape", PACKED_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", fp8_packed_configs())
def test_fp8_packed_config_parity(handle, packed_cases, cfg, shape):
    M, N, K = shape
    c = packed_cases[shape]
    log(f"fp8 packed config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y = forward(handle, c["a8"], c["p8"], M, N, K, c["s"], cfg)
    assert_parity(y, c["y"], f"fp8 packed cfg {cfg} {shape}")


def test_fp8_packed_k_zero_and_errors(handle):
    t = torch()
    M, N = 40, 72
    y = t.full((M, N), -1, dtype=t.int16, device="cuda")
    sw.swiglu_forward_fp8(handle, 0, 0, y, M, N, 0, variant=sw.VARIANT_FP8_PACKED)
    t.cuda.synchronize()
    assert np.all(decode(host(y)) == 0.0)
    assert sw.swiglu_fp8_packed_bytes(N, 144) == ((2 * N + 15) // 16) * 2 * 2048
    assert sw.swiglu_fp8_packed_bytes(N, 0) == 0
    a = t.zeros((M, 144), dtype=t.uint8, device="cuda")
    p = t.zeros((sw.swiglu_fp8_packed_bytes(N, 144),), dtype=t.uint8, device="cuda")
    plain = [i for i in fp8_configs() if variant_of(i) == sw.VARIANT_INTERLEAVE][0]
    with pytest.raises(sw.SwiGLUError) as e:               # a k-major config on P8
        sw.swiglu_forward_fp8(handle, a, p, y, M, N, 144, config_id=plain,
                              variant=sw.VARIANT_FP8_PACKED)
    assert e.value.status == sw.ERR_INVALID_ARG
    w8 = t.zeros((2 * N, 144), dtype=t.uint8, device="cuda")
    with pytest.raises(sw.SwiGLUError) as e:               # N % 8
        sw.swiglu_pack_fp8_fragments(handle, w8, p, 144, 68)
    assert e.value.status == sw.ERR_UNSUPPORTED
    with pytest.raises(sw.SwiGLUError) as e:               # P8 overlaps W8
        sw.swiglu_pack_fp8_fragments(handle, p, p, 144, N)
    assert e.value.status == sw.ERR_INVALID_ARG
