"""GPU parity of the fragment-ordered W_fused path (SWIGLU_LAYOUT_PACKED).

W_fused [K, 2N] ("Riepilogo Tecnico: Sovrapposizione delle Attivazioni a
Livello di Tile...", §Metodologia, Kernel-2) stored in the order the decode
kernel's MFMAs consume it.  The device pack must equal the oracle's pack bit
for bit (padding included), and every packed configuration's forward over
the oracle-packed weights must meet the parity bar against the oracle's
plain definition on the unpacked weights.
"""
import ctypes

import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gpu_util import Run, assert_parity, configs_of, decode, dev, host, log

pytestmark = pytest.mark.gpu

# ragged in every dimension: N not a multiple of 64 (partial slabs), K not a
# multiple of 32 (partial steps), odd and even step counts per wave
SHAPES = [
    (300, 264, 200),
    (37, 136, 520),
    (1, 8, 8),
    (129, 520, 96),
    (33, 72, 40),
    (16, 4864, 896),
    (13, 16504, 72),   # 258 slabs, the last partial: whole slabs on every CU, then quarters
]


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


def _inputs(M, N, K, seed):
    from gemm_epilogues_mlp_amd import inputs as I
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
        a, w1, w2 = _inputs(M, N, K, 300 + i)
        out[(M, N, K)] = dict(a=a, w1=w1, w2=w2, p=oracle.pack_fragments(w1, w2),
                              y=oracle.swiglu_rows(a, w1, w2))
    return out


def test_packed_bytes():
    assert sw.swiglu_packed_bytes(72, 40) == 2 * 2 * 2 * 4096
    assert sw.swiglu_packed_bytes(18944, 3584) == 2 * 296 * 112 * 4096
    assert sw.swiglu_packed_bytes(0, 40) == 0 and sw.swiglu_packed_bytes(8, 0) == 0
    for N, K in ((72, 40), (8, 8), (264, 200)):
        assert sw.swiglu_packed_bytes(N, K) == 2 * oracle.packed_size(N, K)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_device_pack_matches_oracle(handle, cases, shape):
    import torch
    M, N, K = shape
    c = cases[shape]
    log(f"pack_fragments K={K} N={N}")
    p = torch.full((sw.swiglu_packed_bytes(N, K) // 2,), -1, dtype=torch.int16, device="cuda")
    sw.swiglu_pack_fragments(handle, dev(c["w1"]), dev(c["w2"]), p, K, N)
    torch.cuda.synchronize()
    assert np.array_equal(host(p), c["p"])


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", configs_of(sw.VARIANT_PACKED))
def test_packed_config_parity(handle, cases, cfg, shape):
    M, N, K = shape
    c = cases[shape]
    log(f"packed config {cfg} {sw.swiglu_config_info(cfg)} shape {shape}")
    y = Run(handle).fused(dev(c["a"]), dev(c["p"]), None, M, N, K, sw.LAYOUT_PACKED, cfg,
                          sw.VARIANT_PACKED)
    assert_parity(host(y), c["y"], f"packed cfg {cfg} {shape}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_packed_auto_choice(handle, cases, shape):
    """AUTO and the INTERLEAVE variant both run the packed family; the query
    reports it; two runs give identical bits."""
    import torch
    M, N, K = shape
    c = cases[shape]
    v, tile, _ = sw.swiglu_query(handle, M, N, K, sw.LAYOUT_PACKED)
    log(f"packed AUTO {shape} -> variant {v} tile {tile}")
    assert v == sw.VARIANT_PACKED and tile["variant"] == sw.VARIANT_PACKED
    r = Run(handle)
    a, p = dev(c["a"]), dev(c["p"])
    y1 = r.fused(a, p, None, M, N, K, sw.LAYOUT_PACKED)
    y2 = r.fused(a, p, None, M, N, K, sw.LAYOUT_PACKED, -1, sw.VARIANT_INTERLEAVE)
    assert_parity(host(y1), c["y"], f"packed AUTO {shape}")
    assert torch.equal(y1, y2)


def test_packed_k0_writes_zeros(handle):
    import torch
    y = torch.full((5, 72), -1, dtype=torch.int16, device="cuda")
    sw.swiglu_forward(handle, None, None, None, y, 5, 72, 0, sw.LAYOUT_PACKED)
    torch.cuda.synchronize()
    assert (decode(host(y)) == 0).all()


def test_packed_argument_errors(handle):
    import torch
    lib = sw.load()
    M, N, K = 16, 72, 40
    a = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    p = torch.zeros((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16, device="cuda")
    w = torch.zeros((K, N), dtype=torch.int16, device="cuda")
    y = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    h = ctypes.c_void_p(handle)

    def fwd(w2, variant=sw.VARIANT_AUTO, cfg=-1, n=N, k=K):
        return lib.swiglu_forward_ex(h, a.data_ptr(), p.data_ptr(), w2, y.data_ptr(), M, n, k,
                                     sw.LAYOUT_PACKED, variant, cfg, None)

    assert fwd(None) == sw.OK
    assert fwd(w.data_ptr()) == sw.ERR_INVALID_ARG             # W2 must be NULL
    assert fwd(None, sw.VARIANT_SYNC) == sw.ERR_INVALID_ARG      # Kernel-1 order: no
    assert fwd(None, sw.VARIANT_AUTO, 0) == sw.ERR_INVALID_ARG   # config of another family
    assert fwd(None, sw.VARIANT_AUTO, 23) == sw.ERR_INVALID_ARG  # the strided decode kernel
    assert fwd(None, k=36) == sw.ERR_UNSUPPORTED                 # K % 8
    assert lib.swiglu_forward(h, a.data_ptr(), p.data_ptr(), None, y.data_ptr(), M, N, K,
                              3, None) == sw.ERR_INVALID_ARG     # unknown layout
    # pack: N % 8, overlap of P with a source, NULL sources
    assert lib.swiglu_pack_fragments(h, w.data_ptr(), w.data_ptr(), p.data_ptr(), K, 68,
                                     None) == sw.ERR_UNSUPPORTED
    assert lib.swiglu_pack_fragments(h, w.data_ptr(), p.data_ptr(), p.data_ptr(), K, N,
                                     None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_pack_fragments(h, None, w.data_ptr(), p.data_ptr(), K, N,
                                     None) == sw.ERR_INVALID_ARG
    assert lib.swiglu_pack_fragments(h, None, None, None, 0, N, None) == sw.OK
    torch.cuda.synchronize()
