"""GPU parity of every compiled kernel configuration against the CPU oracle,
on seeded shapes that span several tiles and end in ragged tails.

Each output element must satisfy |y - y_ref| <= 0.01 |y_ref| + 2^-10 against
the oracle's unrounded fp32 value; Y is poisoned with NaN before each launch
so an element a kernel forgets to write fails the check.
"""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import Run, assert_parity, configs_of, decode, dev, host, log, rounding_check

pytestmark = pytest.mark.gpu

# (M, N, K): multi-tile with ragged tails for every tile size compiled
SHAPES = [
    (300, 264, 200),   # 2 x 256-row tiles (ragged), 3 x 128-col tiles (ragged), K tail
    (37, 136, 520),    # ragged 16/32/64-row blocks, 3 x 64-col slabs, long K split
    (1, 8, 8),         # single row, single 8-column chunk, one k octet
    (129, 520, 96),    # one row past a tile, N not a multiple of 64
]


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


def _inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = I.f32_to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    s = np.float32(1.0 / np.sqrt(K))
    w1 = I.f32_to_bf16_bits(rng.standard_normal((K, N), dtype=np.float32) * s)
    w2 = I.f32_to_bf16_bits(rng.standard_normal((K, N), dtype=np.float32) * s)
    return a, w1, w2


@pytest.fixture(scope="module")
def cases():
    out = {}
    for i, (M, N, K) in enumerate(SHAPES):
        a, w1, w2 = _inputs(M, N, K, 100 + i)
        wf = I.interleave_columns(w1, w2)
        y_ref, g_ref, u_ref = oracle.swiglu_rows(a, w1, w2, with_gate_up=True)
        out[(M, N, K)] = dict(a=a, w1=w1, w2=w2, wf=wf, y=y_ref, g=g_ref, u=u_ref)
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", configs_of(sw.VARIANT_INTERLEAVE))
def test_interleave_config_parity(handle, cases, cfg, shape):
    M, N, K = shape
    c = cases[shape]
    log(f"interleave config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y = Run(handle).fused(dev(c["a"]), dev(c["wf"]), None, M, N, K, sw.LAYOUT_INTERLEAVED,
                          cfg, sw.VARIANT_INTERLEAVE)
    assert_parity(host(y), c["y"], f"interleave cfg {cfg} {shape}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", configs_of(sw.VARIANT_SYNC))
def test_sync_config_parity(handle, cases, cfg, shape):
    M, N, K = shape
    c = cases[shape]
    log(f"sync config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y = Run(handle).fused(dev(c["a"]), dev(c["w1"]), dev(c["w2"]), M, N, K,
                          sw.LAYOUT_SEPARATE, cfg, sw.VARIANT_SYNC)
    assert_parity(host(y), c["y"], f"sync cfg {cfg} {shape}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", configs_of(sw.VARIANT_GEMM))
def test_unfused_config_parity(handle, cases, cfg, shape):
    """Unfused baseline: G and U against the oracle's fp32 products and as
    their bf16 rounding (up to what the summation order changes), then the
    separate gate kernel against the oracle's gate on those accepted G and U
    (so a rounded intermediate that summation order moved by one bf16 step
    cannot make the check flaky)."""
    M, N, K = shape
    c = cases[shape]
    log(f"unfused gemm config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y, g, u = Run(handle).unfused(dev(c["a"]), dev(c["w1"]), dev(c["w2"]), M, N, K, cfg)
    g, u, y = host(g), host(u), host(y)
    assert_parity(g, c["g"], f"unfused G cfg {cfg} {shape}")
    assert_parity(u, c["u"], f"unfused U cfg {cfg} {shape}")
    rounding_check(g, c["g"], K, f"unfused G rounding cfg {cfg} {shape}")
    rounding_check(u, c["u"], K, f"unfused U rounding cfg {cfg} {shape}")
    y_ref = oracle.gate(oracle.decode_bf16(g), oracle.decode_bf16(u))
    assert_parity(y, y_ref, f"unfused Y cfg {cfg} {shape}")


# The sync family's pair tiles (Gate and Up wave groups over the same A
# k-tiles) sum each output's Gate and Up products in the same order, with the
# same MFMA blocks, as the sync tiles that run the Gate phase and then the Up
# phase: both must give the same Y bit for bit (signed zeros aside).
PAIR_CONFIGS = [89, 90, 91, 92]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_pair_tiles_match_phase_tiles_bitwise(handle, cases, shape):
    M, N, K = shape
    c = cases[shape]
    ref = None
    for cfg in [8] + PAIR_CONFIGS:
        assert sw.swiglu_config_info(cfg)["variant"] == sw.VARIANT_SYNC
        log(f"sync config {cfg} bitwise shape {shape}")
        y = host(Run(handle).fused(dev(c["a"]), dev(c["w1"]), dev(c["w2"]), M, N, K,
                                   sw.LAYOUT_SEPARATE, cfg, sw.VARIANT_SYNC))
        y = np.where(y == np.uint16(0x8000), np.uint16(0), y.astype(np.uint16))
        if ref is None:
            ref = y
        else:
            bad = np.flatnonzero(y != ref)
            assert bad.size == 0, f"config {cfg} differs from config 8 at {bad[:8]} of {shape}"


def _split_configs():
    """bf16 split-tail configurations (the FP8 ones are covered in test_gpu_fp8.py)."""
    return [i for i in range(sw.swiglu_config_count())
            if sw.swiglu_config_info(i)["tail_split"]
            and sw.swiglu_config_info(i)["variant"] in (sw.VARIANT_SYNC, sw.VARIANT_INTERLEAVE,
                                                        sw.VARIANT_GEMM)]


@pytest.mark.parametrize("cfg", _split_configs())
def test_split_tail_parity(handle, cfg):
    """A launch whose tiles fill whole rounds of workgroups (one per CU) plus a
    short last round, which the split-tail configs run as quarter tiles: both
    tile kinds, their boundary in the tile order, and ragged edges in M, N, K."""
    t = __import__("torch")
    info = sw.swiglu_config_info(cfg)
    cus = t.cuda.get_device_properties(0).multi_processor_count
    bm, bn = info["bm"], info["bn"]
    K = 72
    M = 8 * bm - 40                       # 8 tile rows, the last one ragged
    ntn = cus // 8 + 1                    # 8 * ntn tiles: whole rounds plus 8
    N = ntn * bn - 8                      # last tile column ragged
    nt = 8 * ntn
    n_big, tail = nt // cus * cus, nt % cus
    assert n_big > 0 and 0 < 4 * tail <= cus, "shape must exercise both tile kinds"
    a, w1, w2 = _inputs(M, N, K, 777)
    log(f"split-tail config {cfg} {info} shape {(M, N, K)} big {n_big} tail {tail}")
    if info["variant"] == sw.VARIANT_GEMM:
        y, g, u = Run(handle).unfused(dev(a), dev(w1), dev(w2), M, N, K, cfg)
        g_ref = oracle.swiglu_rows(a, w1, w2, with_gate_up=True)[1]
        assert_parity(host(g), g_ref, f"split-tail G cfg {cfg}")
    elif info["variant"] == sw.VARIANT_SYNC:
        y = Run(handle).fused(dev(a), dev(w1), dev(w2), M, N, K, sw.LAYOUT_SEPARATE, cfg,
                              sw.VARIANT_SYNC)
        assert_parity(host(y), oracle.swiglu_rows(a, w1, w2), f"split-tail cfg {cfg}")
    else:
        wf = I.interleave_columns(w1, w2)
        y = Run(handle).fused(dev(a), dev(wf), None, M, N, K, sw.LAYOUT_INTERLEAVED, cfg,
                              sw.VARIANT_INTERLEAVE)
        assert_parity(host(y), oracle.swiglu_rows(a, w1, w2), f"split-tail cfg {cfg}")


@pytest.mark.parametrize("layout", [sw.LAYOUT_SEPARATE, sw.LAYOUT_INTERLEAVED])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_auto_selection_parity(handle, cases, shape, layout):
    M, N, K = shape
    c = cases[shape]
    w1 = c["wf"] if layout == sw.LAYOUT_INTERLEAVED else c["w1"]
    w2 = None if layout == sw.LAYOUT_INTERLEAVED else dev(c["w2"])
    t = __import__("torch")
    y = t.full((M, N), -1, dtype=t.int16, device="cuda")
    sw.swiglu_forward(handle, dev(c["a"]), dev(w1), w2, y, M, N, K, layout)
    t.cuda.synchronize()
    assert_parity(host(y), c["y"], f"auto layout {layout} {shape}")


def test_pack_kernel_bitwise(handle):
    t = __import__("torch")
    for K, N in [(3, 8), (200, 264), (896, 4864)]:
        rng = np.random.default_rng(K * N)
        w1 = rng.integers(0, 65536, (K, N), dtype=np.uint16)
        w2 = rng.integers(0, 65536, (K, N), dtype=np.uint16)
        wf = t.full((K, 2 * N), 0x5555, dtype=t.int16, device="cuda")
        sw.swiglu_pack_interleaved(handle, dev(w1), dev(w2), wf, K, N)
        t.cuda.synchronize()
        assert np.array_equal(host(wf), oracle.pack_interleaved(w1, w2))


def test_k_zero_writes_zeros(handle):
    t = __import__("torch")
    M, N = 40, 72
    for layout in (sw.LAYOUT_SEPARATE, sw.LAYOUT_INTERLEAVED):
        y = t.full((M, N), -1, dtype=t.int16, device="cuda")
        w2 = None if layout == sw.LAYOUT_INTERLEAVED else 0
        sw.swiglu_forward(handle, 0, 0, w2, y, M, N, 0, layout)
        t.cuda.synchronize()
        assert np.all(decode(host(y)) == 0.0)



def _persistent_configs():
    return [i for i in range(sw.swiglu_config_count()) if sw.swiglu_config_info(i)["family"] == 2]


# shapes on which the persistent configurations run their tile loop (K a
# whole number of 128-deep rings, at least two tiles per CU): a quarter-tile
# last round, an unsplit partial last round, ragged M and N, several tiles per
# workgroup
PERSIST_SHAPES = {sw.VARIANT_INTERLEAVE: [(2048, 8960, 128), (4000, 9000, 256), (1280, 30000, 384)],
                  sw.VARIANT_GEMM: [(4000, 8440, 128), (4000, 9400, 256), (2304, 16360, 384)]}


@pytest.mark.parametrize("cfg", _persistent_configs())
def test_persistent_parity(handle, cfg):
    """The persistent tile loop (the next tile's loads under each tile's last
    steps, Y staged through its own LDS region), every output element."""
    from gpu_util import full_check
    info = sw.swiglu_config_info(cfg)
    for i, (M, N, K) in enumerate(PERSIST_SHAPES[info["variant"]]):
        a, w1, w2 = _inputs(M, N, K, 900 + i)
        log(f"persistent config {cfg} shape {(M, N, K)}")
        if info["variant"] == sw.VARIANT_GEMM:
            y, g, u = Run(handle).unfused(dev(a), dev(w1), dev(w2), M, N, K, cfg)
            _, g_ref, u_ref = oracle.swiglu_rows(a, w1, w2, with_gate_up=True)
            full_check(host(g), g_ref, f"persistent G cfg {cfg} {(M, N, K)}")
            full_check(host(u), u_ref, f"persistent U cfg {cfg} {(M, N, K)}")
        else:
            wf = I.interleave_columns(w1, w2)
            y = Run(handle).fused(dev(a), dev(wf), None, M, N, K, sw.LAYOUT_INTERLEAVED, cfg,
                                  sw.VARIANT_INTERLEAVE)
            full_check(host(y), oracle.swiglu_rows(a, w1, w2), f"persistent cfg {cfg} {(M, N, K)}")
