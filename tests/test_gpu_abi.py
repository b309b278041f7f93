"""The C ABI's error contract on the GPU: every rejected call returns its
status synchronously and enqueues nothing (Y keeps its poison)."""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
from gpu_util import configs_of, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    h = sw.swiglu_create(0)
    M, N, K = 64, 64, 64
    t = dict(
        torch=torch, h=h, M=M, N=N, K=K,
        a=torch.zeros((M, K), dtype=torch.int16, device="cuda"),
        w1=torch.zeros((K, N), dtype=torch.int16, device="cuda"),
        w2=torch.zeros((K, N), dtype=torch.int16, device="cuda"),
        wf=torch.zeros((K, 2 * N), dtype=torch.int16, device="cuda"),
        y=torch.full((M, N), -1, dtype=torch.int16, device="cuda"),
    )
    yield t
    sw.swiglu_destroy(h)


def _status(fn, *args):
    try:
        fn(*args)
        return sw.OK
    except sw.SwiGLUError as e:
        return e.status


def test_runtime_is_shared_with_torch(env):
    """One HIP runtime in the process: the library resolved torch's."""
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    log(f"libamdhip64 mapped from: {sorted(libs)}")
    assert len(libs) == 1


def test_create_checks(env):
    import torch
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_create(torch.cuda.device_count() + 3)
    assert e.value.status == sw.ERR_DEVICE
    h = sw.swiglu_create(0)
    sw.swiglu_destroy(h)


def test_invalid_arguments(env):
    e = env
    h, M, N, K = e["h"], e["M"], e["N"], e["K"]
    f = sw.swiglu_forward
    S, IL = sw.LAYOUT_SEPARATE, sw.LAYOUT_INTERLEAVED
    cases = [
        (f, h, e["a"], e["w1"], e["w2"], e["y"], -1, N, K, S),
        (f, h, e["a"], e["w1"], e["w2"], e["y"], M, -8, K, S),
        (f, h, e["a"], e["w1"], e["w2"], e["y"], M, N, -8, S),
        (f, h, None, e["w1"], e["w2"], e["y"], M, N, K, S),
        (f, h, e["a"], None, e["w2"], e["y"], M, N, K, S),
        (f, h, e["a"], e["w1"], None, e["y"], M, N, K, S),
        (f, h, e["a"], e["w1"], e["w2"], None, M, N, K, S),
        (f, h, e["a"], e["wf"], e["w2"], e["y"], M, N, K, IL),   # W2 must be NULL
        (f, h, e["a"], e["w1"], e["w2"], e["y"], M, N, K, 7),    # unknown layout
        (f, h, e["a"], e["w1"], e["w2"], e["a"], M, N, K, S),    # Y aliases A
    ]
    for c in cases:
        assert _status(*c) == sw.ERR_INVALID_ARG, c[6:]
    # variant/layout and config/variant mismatches
    assert _status(sw.swiglu_forward_ex, h, e["a"], e["wf"], None, e["y"], M, N, K, IL,
                   sw.VARIANT_SYNC, -1) == sw.ERR_INVALID_ARG
    sync_cfg = configs_of(sw.VARIANT_SYNC)[0]
    assert _status(sw.swiglu_forward_ex, h, e["a"], e["wf"], None, e["y"], M, N, K, IL,
                   sw.VARIANT_AUTO, sync_cfg) == sw.ERR_INVALID_ARG
    assert _status(sw.swiglu_forward_ex, h, e["a"], e["w1"], e["w2"], e["y"], M, N, K, S,
                   sw.VARIANT_AUTO, 10 ** 6) == sw.ERR_INVALID_ARG
    gemm_cfg = configs_of(sw.VARIANT_GEMM)[0]
    assert _status(sw.swiglu_forward_ex, h, e["a"], e["w1"], e["w2"], e["y"], M, N, K, S,
                   sw.VARIANT_AUTO, gemm_cfg) == sw.ERR_INVALID_ARG
    ws = e["torch"].empty((2, M, N), dtype=e["torch"].int16, device="cuda")
    assert _status(sw.swiglu_forward_unfused, h, e["a"], e["w1"], e["w2"], ws, e["y"], M, N, K,
                   sync_cfg) == sw.ERR_INVALID_ARG
    assert _status(sw.swiglu_forward_unfused, h, e["a"], e["w1"], e["w2"], None, e["y"], M, N,
                   K) == sw.ERR_INVALID_ARG
    e["torch"].cuda.synchronize()
    assert np.all(host(e["y"]) == 0xFFFF), "a rejected call wrote Y"


def test_unsupported_shapes_and_alignment(env):
    e = env
    h, M, N, K = e["h"], e["M"], e["N"], e["K"]
    S = sw.LAYOUT_SEPARATE
    f = sw.swiglu_forward
    assert _status(f, h, e["a"], e["w1"], e["w2"], e["y"], M, N - 4, K, S) == sw.ERR_UNSUPPORTED
    assert _status(f, h, e["a"], e["w1"], e["w2"], e["y"], M, N, K - 4, S) == sw.ERR_UNSUPPORTED
    a_off = e["a"].data_ptr() + 2  # 2-byte aligned only
    assert _status(f, h, a_off, e["w1"], e["w2"], e["y"], M - 1, N, K - 8, S) == \
        sw.ERR_UNSUPPORTED
    assert _status(sw.swiglu_pack_interleaved, h, e["w1"], e["w2"], e["wf"], K, N - 4) == \
        sw.ERR_UNSUPPORTED
    e["torch"].cuda.synchronize()
    assert np.all(host(e["y"]) == 0xFFFF)


def test_tensors_of_2gib_are_rejected(env):
    """Each tensor must stay below 2 GiB (32-bit byte offsets in the kernels):
    a shape over the limit is refused before anything is launched, so the
    small buffers passed here are never touched."""
    e = env
    h = e["h"]
    S, IL = sw.LAYOUT_SEPARATE, sw.LAYOUT_INTERLEAVED
    f = sw.swiglu_forward
    big_m = 1 << 20                                  # A = 2 * 2^20 * 1024 B = 2 GiB
    assert _status(f, h, e["a"], e["w1"], e["w2"], e["y"], big_m, 8, 1024, S) == \
        sw.ERR_UNSUPPORTED
    assert _status(f, h, e["a"], e["w1"], e["w2"], e["y"], 8, 1 << 20, 1024, S) == \
        sw.ERR_UNSUPPORTED                          # W1 = 2 GiB
    assert _status(f, h, e["a"], e["wf"], None, e["y"], 8, 1 << 19, 1024, IL) == \
        sw.ERR_UNSUPPORTED                          # W_fused = 4 * 2^19 * 1024 B = 2 GiB
    assert _status(f, h, e["a"], e["w1"], e["w2"], e["y"], 1 << 20, 1024, 8, S) == \
        sw.ERR_UNSUPPORTED                          # Y = 2 GiB
    e["torch"].cuda.synchronize()
    assert np.all(host(e["y"]) == 0xFFFF), "a rejected call wrote Y"


def test_empty_is_noop(env):
    e = env
    h = e["h"]
    for M, N in ((0, 64), (64, 0)):
        sw.swiglu_forward(h, None, None, None, None, M, N, 64, sw.LAYOUT_SEPARATE)
        sw.swiglu_forward(h, None, None, None, None, M, N, 64, sw.LAYOUT_INTERLEAVED)
        sw.swiglu_forward_unfused(h, None, None, None, None, None, M, N, 64)
    sw.swiglu_pack_interleaved(h, None, None, None, 0, 64)
    e["torch"].cuda.synchronize()


def test_query_reports_a_valid_config(env):
    h = env["h"]
    family = {sw.LAYOUT_SEPARATE: sw.VARIANT_SYNC, sw.LAYOUT_INTERLEAVED: sw.VARIANT_INTERLEAVE,
              sw.LAYOUT_PACKED: sw.VARIANT_PACKED}
    for M in (1, 16, 33, 64, 65, 128, 2048, 8192):
        for layout in family:
            v, tile, rec = sw.swiglu_query(h, M, 4864, 896, layout)
            assert v == family[layout]
            assert tile["variant"] == v
            # fragment-ordered weights up to M = 64, the interleaved layout above
            assert rec == (sw.LAYOUT_PACKED if M <= 64 else sw.LAYOUT_INTERLEAVED)
    # wide matrices (N >= 16384 on 256 CUs): packed only up to M = 16
    for M, rec_want in ((1, sw.LAYOUT_PACKED), (16, sw.LAYOUT_PACKED),
                        (17, sw.LAYOUT_INTERLEAVED), (64, sw.LAYOUT_INTERLEAVED)):
        assert sw.swiglu_query(h, M, 18944, 3584, sw.LAYOUT_SEPARATE)[2] == rec_want
        assert sw.swiglu_query_unfused(h, M, 4864, 896)["variant"] == sw.VARIANT_GEMM
