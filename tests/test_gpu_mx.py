"""GPU parity of the MXFP8 path (OCP Microscaling: E4M3 elements with one E8M0
scale per 32 consecutive k) against the CPU oracle.

* MX quantisation: rows of varied magnitudes, zero, subnormal, infinite and
  NaN blocks, every code and scale bit for bit;
* the bf16 k-major pairing W1, W2 [K, N] -> Wt [2N, K]: bit for bit;
* the forward, every MX configuration on seeded shapes with ragged tails in M
  and N (K a multiple of 64), a split-tail launch, and the five Qwen2.5-shaped
  workloads at full size (every element of Y against the oracle's full Y);
  at full size the device's pack and quantiser also reproduce the oracle's
  bits.  Bar: |y - y_ref| <=
  0.01 |y_ref| + 2^-10 against the oracle's value for the same codes and scales.

Input recipe: the seeded bf16 draws of the bf16 tests (A ~ N(0, 1),
W ~ N(0, 1/K)); A's rows and the rows of the k-major pairing of W1, W2 are
quantised by the oracle's MX quantiser.
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


def dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch().from_numpy(x).cuda()


def mx_inputs(a_bits, w1_bits, w2_bits):
    """Oracle MX quantisation of A's rows and of the k-major paired weights."""
    qa, sa = oracle.quantize_mx(I.bf16_bits_to_f32(a_bits))
    wt = oracle.pack_kmajor_bf16(w1_bits, w2_bits)
    qw, sw_ = oracle.quantize_mx(I.bf16_bits_to_f32(wt))
    return qa, sa, qw, sw_, wt


def forward(handle, qa, sa, qw, sw_, M, N, K, cfg=-1):
    t = torch()
    y = empty_poisoned((M, N))
    sw.swiglu_forward_mx(handle, dev(qa), dev(sa), dev(qw), dev(sw_), y, M, N, K, sa.shape[1],
                         config_id=cfg)
    t.cuda.synchronize()
    return host(y)


# --------------------------------------------------------------------------- quantise
def test_quantize_mx_bitwise(handle):
    t = torch()
    rng = np.random.default_rng(21)
    R, K = 64, 256
    x = rng.standard_normal((R, K)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-6, 6, (R, 1))).astype(np.float32)      # rows of every magnitude
    x[1, :32] = 0.0                                                  # a zero block
    x[2, 32:64] = np.float32(2.0 ** -130)                            # a subnormal block
    x[3, 5] = np.inf                                                 # an infinity
    x[4, 70] = np.nan                                                # a NaN
    x[5, 100] = -448.0 * 2.0 ** 20                                   # an exact block maximum
    bits = I.f32_to_bf16_bits(x)
    ks = oracle.mx_scale_stride(K)
    q = t.full((R, K), 0x55, dtype=t.uint8, device="cuda")
    s = t.full((R, ks), 0x55, dtype=t.uint8, device="cuda")
    sw.swiglu_quantize_mx(handle, dev(bits), q, s, R, K, ks)
    t.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_mx(I.bf16_bits_to_f32(bits), ks)
    got_q, got_s = q.cpu().numpy(), s.cpu().numpy()
    assert np.array_equal(got_s, s_ref)
    nan = np.isnan(I.bf16_bits_to_f32(bits))
    assert np.all((got_q[nan] & 0x7F) == 0x7F)                       # NaN code of either sign
    assert np.array_equal(got_q[~nan], q_ref[~nan])


def test_pack_kmajor_bitwise(handle):
    t = torch()
    rng = np.random.default_rng(22)
    for K, N in [(8, 8), (200, 264), (1536, 8960)]:
        w1 = rng.integers(0, 65536, (K, N), dtype=np.uint16)
        w2 = rng.integers(0, 65536, (K, N), dtype=np.uint16)
        wt = t.full((2 * N, K), 0x5555, dtype=t.int16, device="cuda")
        sw.swiglu_pack_kmajor(handle, dev(w1), dev(w2), wt, K, N)
        t.cuda.synchronize()
        assert np.array_equal(host(wt), oracle.pack_kmajor_bf16(w1, w2))


def test_mx_errors(handle):
    t = torch()
    M, N, K = 40, 72, 96
    a = t.zeros((M, K), dtype=t.uint8, device="cuda")
    w = t.zeros((2 * N, K), dtype=t.uint8, device="cuda")
    s = t.zeros((2 * N, 16), dtype=t.uint8, device="cuda")
    y = t.zeros((M, N), dtype=t.int16, device="cuda")
    with pytest.raises(sw.SwiGLUError) as e:                         # K % 64 != 0
        sw.swiglu_forward_mx(handle, a, s, w, s, y, M, N, K, 16)
    assert e.value.status == sw.ERR_UNSUPPORTED
    with pytest.raises(sw.SwiGLUError) as e:                         # ks < K / 32
        sw.swiglu_forward_mx(handle, a, s, w, s, y, M, N, 64, 1)
    assert e.value.status == sw.ERR_INVALID_ARG
    with pytest.raises(sw.SwiGLUError) as e:                         # ks % 16 != 0
        sw.swiglu_forward_mx(handle, a, s, w, s, y, M, N, 64, 8)
    assert e.value.status == sw.ERR_UNSUPPORTED
    with pytest.raises(sw.SwiGLUError) as e:                         # a per-tensor FP8 config
        sw.swiglu_forward_mx(handle, a, s, w, s, y, M, N, 64, 16, config_id=43)
    assert e.value.status == sw.ERR_INVALID_ARG
    y.fill_(-1)
    sw.swiglu_forward_mx(handle, 0, 0, 0, 0, y, M, N, 0, 0)          # K = 0: zeros
    t.cuda.synchronize()
    assert np.all(decode(host(y)) == 0.0)


# --------------------------------------------------------------------------- forward
SHAPES = [
    (300, 264, 256),   # ragged 256-row and 128-column tiles, two scale groups
    (37, 136, 576),    # ragged 64-row tiles, K = 9 steps (a partial scale group)
    (1, 8, 64),        # one row, one 8-column chunk, one step
    (129, 520, 128),   # one row past a tile
    (130, 264, 1088),  # 17 steps: three scale groups per phase, the last partial
]


def mx_configs():
    """MX configurations of both kernel orders (the same W8 and scales)."""
    return [i for i in range(sw.swiglu_config_count())
            if sw.swiglu_config_info(i)["variant"] in (sw.VARIANT_MXFP8, sw.VARIANT_MXFP8_SYNC)]


@pytest.fixture(scope="module")
def cases():
    out = {}
    for i, (M, N, K) in enumerate(SHAPES):
        a, w1, w2 = I.make_inputs(M, K, N, 50 + i)
        qa, sa, qw, sw_, _ = mx_inputs(a, w1, w2)
        out[(M, N, K)] = dict(q=(qa, sa, qw, sw_), y=oracle.swiglu_mx_rows(qa, sa, qw, sw_))
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", mx_configs())
def test_mx_config_parity(handle, cases, cfg, shape):
    M, N, K = shape
    c = cases[shape]
    log(f"mx config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y = forward(handle, *c["q"], M, N, K, cfg)
    assert_parity(y, c["y"], f"mx cfg {cfg} {shape}")


@pytest.mark.parametrize("cfg", mx_configs())
def test_mx_scale_row_padding_is_not_used(handle, cases, cfg):
    """Scale bytes past K/32 (the row padding up to ks) hold the NaN code 255
    here; the result must not change (the sync order's Gate phase runs zero
    padding steps, whose scales must not come from those bytes)."""
    M, N, K = 130, 264, 1088  # 17 steps: 34 scale bytes a row, ks = 48
    qa, sa, qw, sw_ = cases[(M, N, K)]["q"]
    sa2, sw2 = sa.copy(), sw_.copy()
    assert sa2.shape[1] > K // 32
    sa2[:, K // 32:] = 255
    sw2[:, K // 32:] = 255
    y = forward(handle, qa, sa2, qw, sw2, M, N, K, cfg)
    assert_parity(y, cases[(M, N, K)]["y"], f"mx cfg {cfg}, NaN codes in the scale-row padding")


@pytest.mark.parametrize("cfg", [i for i in mx_configs() if sw.swiglu_config_info(i)["tail_split"]])
def test_mx_split_tail_parity(handle, cfg):
    info = sw.swiglu_config_info(cfg)
    cus = torch().cuda.get_device_properties(0).multi_processor_count
    bm, bn = info["bm"], info["bn"]
    M, ntn, K = 8 * bm - 40, cus // 8 + 1, 128
    N = ntn * bn - 8
    nt = 8 * ntn
    assert nt // cus > 0 and 0 < 4 * (nt % cus) <= cus
    a, w1, w2 = I.make_inputs(M, K, N, 77)
    qa, sa, qw, sw_, _ = mx_inputs(a, w1, w2)
    log(f"mx split-tail config {cfg} shape {(M, N, K)}")
    y = forward(handle, qa, sa, qw, sw_, M, N, K, cfg)
    assert_parity(y, oracle.swiglu_mx_rows(qa, sa, qw, sw_), f"mx split cfg {cfg}")


@pytest.mark.parametrize("order", ["interleave", "sync"])
def test_mx_block_scales_matter(handle, order):
    """Changing one Up block scale of one column changes exactly that column
    (and one Gate block scale, in a later scale group, likewise), in both
    kernel orders."""
    M, N, K = 64, 128, 768
    cfg = -1 if order == "interleave" else \
        sw.swiglu_query_fp8(handle, M, N, K, sw.VARIANT_MXFP8_SYNC)["id"]
    a, w1, w2 = I.make_inputs(M, K, N, 88)
    qa, sa, qw, sw_, _ = mx_inputs(a, w1, w2)
    y0 = forward(handle, qa, sa, qw, sw_, M, N, K, cfg)
    for row, blk, col in [(2 * 5 + 1, 3, 5), (2 * 9, 20, 9)]:       # Up of column 5, Gate of 9
        sw2 = sw_.copy()
        sw2[row, blk] += 2                                           # that k block x4
        y1 = forward(handle, qa, sa, qw, sw2, M, N, K, cfg)
        assert_parity(y1, oracle.swiglu_mx_rows(qa, sa, qw, sw2), f"mx {order} modified scale")
        changed = np.any(y0 != y1, axis=0)
        assert changed[col] and not np.any(np.delete(changed, col))


# --------------------------------------------------------------------------- workloads
@pytest.fixture(scope="module", params=I.WORKLOADS, ids=lambda w: w.name)
def workload(request):
    w = request.param
    log(f"mx inputs for {w.name} M={w.M} K={w.K} N={w.N}")
    a, w1, w2 = I.workload_inputs(w)
    qa, sa, qw, sw_, wt = mx_inputs(a, w1, w2)
    t0 = time.perf_counter()
    y_ref = oracle.swiglu_mx_rows(qa, sa, qw, sw_)
    log(f"mx {w.name}: oracle full Y in {time.perf_counter() - t0:.1f} s")
    return dict(w=w, a=a, w1=w1, w2=w2, wt=wt, q=(qa, sa, qw, sw_), y_ref=y_ref)


def test_mx_workload_parity(handle, workload):
    d = workload
    w = d["w"]
    log(f"mx {w.name}: config {sw.swiglu_query_fp8(handle, w.M, w.N, w.K, sw.VARIANT_MXFP8)['id']}")
    y = forward(handle, *d["q"], w.M, w.N, w.K)
    s = full_check(y, d["y_ref"], f"mx {w.name}")
    log(f"mx {w.name}: all {s['elements']} elements within the bar (worst "
        f"{s['worst_frac']:.3f}); share > 1 % off: {s['rel_gt_1pct']:.2e}")


def test_mx_sync_workload_parity(handle, workload):
    """The sync (Kernel-1) order on the same W8 and scales, the table's choice
    for the shape, every output element."""
    d = workload
    w = d["w"]
    cfg = sw.swiglu_query_fp8(handle, w.M, w.N, w.K, sw.VARIANT_MXFP8_SYNC)["id"]
    log(f"mx sync {w.name}: config {cfg}")
    y = forward(handle, *d["q"], w.M, w.N, w.K, cfg)
    s = full_check(y, d["y_ref"], f"mx sync {w.name}")
    log(f"mx sync {w.name}: all {s['elements']} elements within the bar (worst "
        f"{s['worst_frac']:.3f}); share > 1 % off: {s['rel_gt_1pct']:.2e}")


def test_mx_workload_device_pipeline_matches(handle, workload):
    """The device's k-major pack and MX quantiser reproduce the oracle's bits
    for the full-size weights and activations."""
    t = torch()
    d = workload
    w = d["w"]
    K, N, M = w.K, w.N, w.M
    ks = oracle.mx_scale_stride(K)
    wt = t.empty((2 * N, K), dtype=t.int16, device="cuda")
    sw.swiglu_pack_kmajor(handle, dev(d["w1"]), dev(d["w2"]), wt, K, N)
    q = t.empty((2 * N, K), dtype=t.uint8, device="cuda")
    s = t.empty((2 * N, ks), dtype=t.uint8, device="cuda")
    sw.swiglu_quantize_mx(handle, wt, q, s, 2 * N, K, ks)
    qa = t.empty((M, K), dtype=t.uint8, device="cuda")
    sa = t.empty((M, ks), dtype=t.uint8, device="cuda")
    sw.swiglu_quantize_mx(handle, dev(d["a"]), qa, sa, M, K, ks)
    t.cuda.synchronize()
    assert np.array_equal(host(wt), d["wt"])
    assert np.array_equal(q.cpu().numpy(), d["q"][2]) and np.array_equal(s.cpu().numpy(), d["q"][3])
    assert np.array_equal(qa.cpu().numpy(), d["q"][0]) and np.array_equal(sa.cpu().numpy(), d["q"][1])


# --------------------------------------------------------------------------- fragment order
def mx_packed_configs():
    return [i for i in range(sw.swiglu_config_count())
            if sw.swiglu_config_info(i)["variant"] == sw.VARIANT_MXFP8_PACKED]


def forward_packed(handle, qa, sa, p8, sw_, M, N, K, cfg=-1):
    t = torch()
    y = empty_poisoned((M, N))
    sw.swiglu_forward_mx_packed(handle, dev(qa), dev(sa), dev(p8), dev(sw_), y, M, N, K,
                                sa.shape[1], config_id=cfg)
    t.cuda.synchronize()
    return host(y)


# the tile shapes plus a row count past 32, many 16-step scale groups and a
# partial one, and the 0.5B shape at a decode-sized M
PACKED_SHAPES = SHAPES + [(33, 72, 1088), (16, 4864, 896)]


@pytest.fixture(scope="module")
def packed_cases():
    out = {}
    for i, (M, N, K) in enumerate(PACKED_SHAPES):
        a, w1, w2 = I.make_inputs(M, K, N, 60 + i)
        qa, sa, qw, sw_, _ = mx_inputs(a, w1, w2)
        out[(M, N, K)] = dict(qa=qa, sa=sa, qw=qw, sw=sw_, p8=oracle.pack_mx_fragments(qw),
                              y=oracle.swiglu_mx_rows(qa, sa, qw, sw_))
    return out


@pytest.mark.parametrize("shape", PACKED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mx_fragment_pack_bitwise(handle, packed_cases, shape):
    t = torch()
    M, N, K = shape
    c = packed_cases[shape]
    p8 = t.full((sw.swiglu_mx_packed_bytes(N, K),), 0x55, dtype=t.uint8, device="cuda")
    sw.swiglu_pack_mx_fragments(handle, dev(c["qw"]), p8, K, N)
    t.cuda.synchronize()
    assert np.array_equal(p8.cpu().numpy(), c["p8"])


@pytest.mark.parametrize("shape", PACKED_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", mx_packed_configs())
def test_mx_packed_config_parity(handle, packed_cases, cfg, shape):
    M, N, K = shape
    c = packed_cases[shape]
    log(f"mx packed config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y = forward_packed(handle, c["qa"], c["sa"], c["p8"], c["sw"], M, N, K, cfg)
    assert_parity(y, c["y"], f"mx packed cfg {cfg} {shape}")


def test_mx_packed_block_scales_matter(handle):
    """Changing one Up block scale of one column changes exactly that column."""
    M, N, K = 16, 128, 256
    a, w1, w2 = I.make_inputs(M, K, N, 89)
    qa, sa, qw, sw_, _ = mx_inputs(a, w1, w2)
    p8 = oracle.pack_mx_fragments(qw)
    sw2 = sw_.copy()
    sw2[2 * 5 + 1, 3] += 2
    y0 = forward_packed(handle, qa, sa, p8, sw_, M, N, K)
    y1 = forward_packed(handle, qa, sa, p8, sw2, M, N, K)
    assert_parity(y1, oracle.swiglu_mx_rows(qa, sa, qw, sw2), "mx packed modified scale")
    changed = np.any(y0 != y1, axis=0)
    assert changed[5] and not np.any(np.delete(changed, 5))


def test_mx_packed_k_zero_and_errors(handle):
    t = torch()
    M, N = 40, 72
    y = t.full((M, N), -1, dtype=t.int16, device="cuda")
    sw.swiglu_forward_mx_packed(handle, 0, 0, 0, 0, y, M, N, 0, 0)
    t.cuda.synchronize()
    assert np.all(decode(host(y)) == 0.0)
    a = t.zeros((M, 128), dtype=t.uint8, device="cuda")
    s = t.zeros((M, 16), dtype=t.uint8, device="cuda")
    p = t.zeros((sw.swiglu_mx_packed_bytes(N, 128),), dtype=t.uint8, device="cuda")
    ws = t.zeros((2 * N, 16), dtype=t.uint8, device="cuda")
    with pytest.raises(sw.SwiGLUError) as e:               # a k-major MX config on P8
        sw.swiglu_forward_mx_packed(handle, a, s, p, ws, y, M, N, 128, 16,
                                    config_id=mx_configs()[0])
    assert e.value.status == sw.ERR_INVALID_ARG
    with pytest.raises(sw.SwiGLUError) as e:               # K % 64
        sw.swiglu_pack_mx_fragments(handle, a, p, 96, N)
    assert e.value.status == sw.ERR_UNSUPPORTED
    with pytest.raises(sw.SwiGLUError) as e:               # P8 overlaps W8
        sw.swiglu_pack_mx_fragments(handle, p, p, 128, N)
    assert e.value.status == sw.ERR_INVALID_ARG


def test_mx_packed_workload_parity(handle, workload):
    d = workload
    w = d["w"]
    qa, sa, qw, sw_ = d["q"]
    cfg = sw.swiglu_query_fp8(handle, w.M, w.N, w.K, sw.VARIANT_MXFP8_PACKED)
    log(f"mx packed {w.name}: config {cfg['id']}")
    p8 = oracle.pack_mx_fragments(qw)
    y = forward_packed(handle, qa, sa, p8, sw_, w.M, w.N, w.K)
    s = full_check(y, d["y_ref"], f"mx packed {w.name}")
    log(f"mx packed {w.name}: all {s['elements']} elements within the bar (worst "
        f"{s['worst_frac']:.3f})")
