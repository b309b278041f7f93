"""The unfused baseline's no-allocation entry point, swiglu_forward_unfused_static,
through the C ABI: its output must equal that of swiglu_forward_unfused (the
same launches on a caller workspace) on consecutive calls of decreasing size,
including a shape whose Gate and Up fill the fixed scratch exactly, and a
shape one row past it must be refused with nothing written.  Both results are
also held to the parity bar against the oracle's unfused emulation."""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import dev, empty_poisoned, full_check, host, log, rounding_check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


def _both(handle, M, N, K, seed):
    import torch
    a, w1, w2 = I.make_inputs(M, K, N, seed)
    A, W1, W2 = dev(a), dev(w1), dev(w2)
    ws = torch.full((2, M, N), -1, dtype=torch.int16, device="cuda")
    y_ws = empty_poisoned((M, N))
    sw.swiglu_forward_unfused(handle, A, W1, W2, ws, y_ws, M, N, K)
    y_st = empty_poisoned((M, N))
    sw.swiglu_forward_unfused_static(handle, A, W1, W2, y_st, M, N, K)
    torch.cuda.synchronize()
    return a, w1, w2, host(ws[0]), host(ws[1]), host(y_ws), host(y_st)


@pytest.mark.parametrize("shapes", [
    [(300, 264, 200, 71), (37, 136, 520, 72)],          # several tiles, then a smaller ragged call
    [(2048, 8960, 1536, 2), (128, 4864, 896, 1)],       # the 1.5B and 0.5B MLP workloads
], ids=["ragged", "workloads"])
def test_static_matches_workspace_entry_point(handle, shapes):
    for (M, N, K, seed) in shapes:
        log(f"unfused_static M={M} N={N} K={K}")
        a, w1, w2, g, u, y_ws, y_st = _both(handle, M, N, K, seed)
        assert np.array_equal(y_st, y_ws), "static-scratch output differs from the workspace one"
        _, g_ref, u_ref = oracle.swiglu_rows(a, w1, w2, with_gate_up=True)
        rounding_check(g, g_ref, K, "G")
        rounding_check(u, u_ref, K, "U")
        full_check(y_st, oracle.gate(oracle.decode_bf16(g), oracle.decode_bf16(u)),
                   f"unfused_static {M}x{N}x{K}")


def test_static_scratch_limit(handle):
    import torch
    # Gate and Up of 4096 x 8192 outputs fill the scratch exactly
    M, N, K = 4096, 8192, 64
    assert 4 * M * N == sw.STATIC_SCRATCH_BYTES
    a, w1, w2, g, u, y_ws, y_st = _both(handle, M, N, K, 73)
    assert np.array_equal(y_st, y_ws)
    rows = np.array([0, 1, M // 2, M - 1])
    _, g_ref, u_ref = oracle.swiglu_rows(a, w1, w2, rows=rows, with_gate_up=True)
    rounding_check(g[rows], g_ref, K, "G at the limit")
    rounding_check(u[rows], u_ref, K, "U at the limit")
    # one row more does not fit: refused before anything is enqueued
    M1 = M + 1
    a1, w1b, w2b = I.make_inputs(M1, K, N, 74)
    y = empty_poisoned((M1, N))
    with pytest.raises(sw.SwiGLUError) as e:
        sw.swiglu_forward_unfused_static(handle, dev(a1), dev(w1b), dev(w2b), y, M1, N, K)
    assert e.value.status == sw.ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert np.all(host(y) == 0xFFFF), "a refused call wrote to Y"
