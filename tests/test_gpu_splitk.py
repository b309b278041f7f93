"""GPU parity of the decode forward with K split over workgroups
(swiglu_forward_packed_splitk): fp32 partial sums of each slab part handed
from S workgroups to the last of them, which adds them in K order before
SiLU and the pair product ("Riepilogo Tecnico: Sovrapposizione delle
Attivazioni a Livello di Tile...", §Risultati: the cross-tile sums kept in
FP32).  Every output element is checked against the oracle's plain
definition on the unpacked weights, for every configuration and a range of
splits (1, ragged, more pieces than K steps), and the workspace's counters
must be back at zero after every call."""
import ctypes

import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gpu_util import assert_parity, configs_of, decode, dev, host, log

pytestmark = pytest.mark.gpu

# M <= 16; ragged N (partial slabs), K not a multiple of 32 (partial steps),
# a narrow N with few slabs (one GPU's share of the 7B MLP under 8-way tensor
# parallelism) and the 7B decode shape itself
SHAPES = [
    (1, 136, 520),
    (7, 72, 40),
    (16, 8, 8),
    (13, 264, 200),
    (16, 2368, 3584),
    (16, 18944, 3584),
]
SPLITS = [1, 2, 3, 5, 64]


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
        a, w1, w2 = _inputs(M, N, K, 700 + i)
        out[(M, N, K)] = dict(a=dev(a), p=dev(oracle.pack_fragments(w1, w2)),
                              y=oracle.swiglu_rows(a, w1, w2))
    return out


def _workspace(N, K, S):
    import torch
    n = sw.swiglu_packed_splitk_workspace_bytes(N, K, S)
    assert n > 0
    return torch.zeros((n,), dtype=torch.uint8, device="cuda")


def _counters_zero(ws, N):
    slabs = (2 * N + 127) // 128
    return int(ws[:slabs * 16].count_nonzero().item()) == 0


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("cfg", configs_of(sw.VARIANT_PACKED_SPLITK))
def test_splitk_parity(handle, cases, cfg, shape):
    import torch
    M, N, K = shape
    c = cases[shape]
    ws = _workspace(N, K, max(SPLITS))
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    for S in SPLITS:
        log(f"split-K config {cfg} S={S} shape {shape}")
        y.fill_(-1)
        sw.swiglu_forward_packed_splitk(handle, c["a"], c["p"], y, M, N, K, ws, ksplit=S,
                                        config_id=cfg)
        torch.cuda.synchronize()
        assert_parity(host(y), c["y"], f"split-K cfg {cfg} S {S} {shape}")
        assert _counters_zero(ws, N), f"counters not reset (cfg {cfg} S {S} {shape})"


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_splitk_plan_and_repeat(handle, cases, shape):
    """The plan's choice meets the bar; calls repeated on one workspace give
    identical bits (the sum of the partials is in a fixed order)."""
    import torch
    M, N, K = shape
    c = cases[shape]
    cfg, S = sw.swiglu_packed_splitk_plan(handle, M, N, K)
    log(f"split-K plan {shape} -> config {cfg}, S = {S}")
    assert sw.swiglu_config_info(cfg)["variant"] == sw.VARIANT_PACKED_SPLITK and 1 <= S <= 64
    ws = _workspace(N, K, S)
    ys = []
    for _ in range(3):
        y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
        sw.swiglu_forward_packed_splitk(handle, c["a"], c["p"], y, M, N, K, ws)
        ys.append(y)
    torch.cuda.synchronize()
    assert_parity(host(ys[0]), c["y"], f"split-K plan {shape}")
    assert torch.equal(ys[0], ys[1]) and torch.equal(ys[0], ys[2])
    assert _counters_zero(ws, N)


def test_splitk_k0_writes_zeros(handle):
    import torch
    M, N = 5, 72
    ws = _workspace(N, 0, 3)
    y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    sw.swiglu_forward_packed_splitk(handle, None, None, y, M, N, 0, ws, ksplit=3)
    torch.cuda.synchronize()
    assert (decode(host(y)) == 0).all() and _counters_zero(ws, N)


def test_splitk_argument_errors(handle):
    import torch
    lib = sw.load()
    M, N, K = 16, 72, 40
    a = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    p = torch.zeros((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16, device="cuda")
    y = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    need = sw.swiglu_packed_splitk_workspace_bytes(N, K, 4)
    ws = torch.zeros((need + 16,), dtype=torch.uint8, device="cuda")
    h = ctypes.c_void_p(handle)

    def fwd(m=M, cfg=-1, S=4, w=ws.data_ptr(), wb=need, yp=y.data_ptr()):
        return lib.swiglu_forward_packed_splitk(h, a.data_ptr(), p.data_ptr(), yp, m, N, K, cfg,
                                                S, w, wb, None)

    assert fwd() == sw.OK
    assert fwd(m=17) == sw.ERR_UNSUPPORTED                     # decode rows only
    assert fwd(cfg=65) == sw.ERR_INVALID_ARG                   # a config of another variant
    assert fwd(S=65) == sw.ERR_UNSUPPORTED                     # at most 64 pieces
    assert fwd(wb=need - 1) == sw.ERR_INVALID_ARG              # workspace too small
    assert fwd(w=None) == sw.ERR_INVALID_ARG
    assert fwd(w=ws.data_ptr() + 8) == sw.ERR_UNSUPPORTED      # not 16-byte aligned
    assert fwd(w=y.data_ptr(), wb=1 << 30) == sw.ERR_INVALID_ARG  # overlaps Y
    assert fwd(m=0) == sw.OK                                   # nothing to do
    assert lib.swiglu_forward_packed_splitk(None, a.data_ptr(), p.data_ptr(), y.data_ptr(), M,
                                            N, K, -1, 4, ws.data_ptr(), need,
                                            None) == sw.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert _counters_zero(ws, N)
