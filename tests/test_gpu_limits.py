"""The largest tensors the kernels take: each just under the 2 GiB limit the
32-bit byte offsets allow (tensors of 2 GiB or more are refused, see
test_gpu_abi), through the table's configurations for both layouts and the
unfused baseline.  Inputs are drawn on the GPU (seeded); sampled output rows
are checked against the oracle."""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gpu_util import assert_parity, host, log

pytestmark = pytest.mark.gpu

# (M, N, K): A = 2MK bytes or W_fused = 4KN bytes is 2^31 - 2^20
CASES = [(65536, 64, 16376), (16, 32768, 16376), (256, 32768, 16376)]


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


def _bf16(t, shape, scale, g):
    return (t.randn(shape, device="cuda", generator=g) * scale).to(t.bfloat16).view(t.int16)


@pytest.mark.parametrize("shape", CASES, ids=lambda s: "x".join(map(str, s)))
def test_largest_tensors(handle, shape):
    import torch as t
    M, N, K = shape
    assert max(2 * M * K, 4 * K * N) < 2 ** 31 <= max(2 * M * K, 4 * K * N) + 2 ** 21
    log(f"limit shape M={M} N={N} K={K}")
    g = t.Generator(device="cuda").manual_seed(M + N + K)
    a, w1, w2 = _bf16(t, (M, K), 1.0, g), _bf16(t, (K, N), K ** -0.5, g), \
        _bf16(t, (K, N), K ** -0.5, g)
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 2)])
    a_h = host(a[t.from_numpy(rows).cuda()])
    w1_h, w2_h = host(w1), host(w2)
    y_ref, g_ref, u_ref = oracle.swiglu_rows(a_h, w1_h, w2_h, with_gate_up=True)

    y = t.full((M, N), -1, dtype=t.int16, device="cuda")
    sw.swiglu_forward(handle, a, w1, w2, y, M, N, K, sw.LAYOUT_SEPARATE)
    t.cuda.synchronize()
    assert_parity(host(y)[rows], y_ref, f"separate {shape}")

    ws = t.full((2, M, N), -1, dtype=t.int16, device="cuda")
    y.fill_(-1)
    sw.swiglu_forward_unfused(handle, a, w1, w2, ws, y, M, N, K)
    t.cuda.synchronize()
    assert_parity(host(ws[0])[rows], g_ref, f"unfused G {shape}")
    assert_parity(host(ws[1])[rows], u_ref, f"unfused U {shape}")
    del ws

    wf = t.empty((K, 2 * N), dtype=t.int16, device="cuda")
    sw.swiglu_pack_interleaved(handle, w1, w2, wf, K, N)
    del w1, w2
    y.fill_(-1)
    sw.swiglu_forward(handle, a, wf, None, y, M, N, K, sw.LAYOUT_INTERLEAVED)
    t.cuda.synchronize()
    assert_parity(host(y)[rows], y_ref, f"interleaved {shape}")
