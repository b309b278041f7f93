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


# fragment-ordered W_fused just under 2 GiB: 511 slabs x 512 steps x 8 KB
@pytest.mark.parametrize("M", [16, 40])
def test_largest_packed_weights(handle, M):
    import torch as t
    N, K = 32704, 16376
    pbytes = sw.swiglu_packed_bytes(N, K)
    assert pbytes < 2 ** 31 <= pbytes + 2 ** 23
    log(f"packed limit M={M} N={N} K={K} ({pbytes} bytes)")
    g = t.Generator(device="cuda").manual_seed(M + 7)
    a, w1, w2 = _bf16(t, (M, K), 1.0, g), _bf16(t, (K, N), K ** -0.5, g), \
        _bf16(t, (K, N), K ** -0.5, g)
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 2)])
    y_ref = oracle.swiglu_rows(host(a[t.from_numpy(rows).cuda()]), host(w1), host(w2))
    p = t.empty((pbytes // 2,), dtype=t.int16, device="cuda")
    sw.swiglu_pack_fragments(handle, w1, w2, p, K, N)
    del w1, w2
    y = t.full((M, N), -1, dtype=t.int16, device="cuda")
    sw.swiglu_forward(handle, a, p, None, y, M, N, K, sw.LAYOUT_PACKED)
    t.cuda.synchronize()
    assert_parity(host(y)[rows], y_ref, f"packed M={M}")
    del p, y


# fragment-ordered W8 just under 2 GiB: 4096 row blocks x 255 steps x 2 KB
def test_largest_fp8_packed_weights(handle):
    import torch as t
    M, N, K = 16, 32768, 32640
    pbytes = sw.swiglu_fp8_packed_bytes(N, K)
    assert pbytes < 2 ** 31 <= pbytes + 2 ** 23 and 2 * N * K < 2 ** 31
    log(f"fp8 packed limit M={M} N={N} K={K} ({pbytes} bytes)")
    rng = np.random.default_rng(11)
    # finite E4M3 codes of both signs, magnitudes up to 0.25 (code 0x28) so sums stay small
    codes = lambda shape: (rng.integers(0, 0x29, shape, dtype=np.uint8) |
                           (rng.integers(0, 2, shape, dtype=np.uint8) << 7))
    a8, w18, w28 = codes((M, K)), codes((K, N)), codes((K, N))
    scales = (1.0, 2.0 ** -4, 2.0 ** -4)
    rows = np.array([0, 5, M - 1])
    y_ref = oracle.swiglu_fp8_rows(a8, w18, w28, *scales, rows=rows)
    w8 = t.empty((2 * N, K), dtype=t.uint8, device="cuda")
    d1, d2 = t.from_numpy(w18).cuda(), t.from_numpy(w28).cuda()
    sw.swiglu_pack_fp8(handle, d1, d2, w8, K, N)
    del d1, d2
    p8 = t.empty((pbytes,), dtype=t.uint8, device="cuda")
    sw.swiglu_pack_fp8_fragments(handle, w8, p8, K, N)
    del w8
    y = t.full((M, N), -1, dtype=t.int16, device="cuda")
    sw.swiglu_forward_fp8(handle, t.from_numpy(a8).cuda(), p8, y, M, N, K, *scales,
                          variant=sw.VARIANT_FP8_PACKED)
    t.cuda.synchronize()
    assert_parity(host(y)[rows], y_ref, "fp8 packed limit")
    del p8, y


# FP8 and MXFP8 activations just under 2 GiB (A8 = M K bytes), through the
# k-major tiles of both orders: the split 256-row tile of each order and the
# table's own choice.  Codes are drawn on the GPU; sampled rows go to the oracle.
def test_largest_fp8_and_mx_activations(handle):
    import torch as t
    M, N, K = 65536, 64, 32704
    assert M * K < 2 ** 31 <= M * K + 2 ** 23 and K % 64 == 0
    log(f"fp8 / mx activation limit M={M} N={N} K={K}")
    g = t.Generator(device="cuda").manual_seed(29)
    # finite E4M3 codes of both signs, magnitudes up to 0.25 (code 0x28)
    codes = lambda shape: (t.randint(0, 0x29, shape, device="cuda", generator=g, dtype=t.uint8) |
                           (t.randint(0, 2, shape, device="cuda", generator=g, dtype=t.uint8) << 7))
    h8 = lambda x: x.cpu().numpy()  # uint8 tensor -> numpy (host() views as bf16 bits)
    a8 = codes((M, K))
    w18, w28 = codes((K, N)), codes((K, N))
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(K).integers(0, M, 2)])
    a8_rows = h8(a8[t.from_numpy(rows).cuda()])
    w18_h, w28_h = h8(w18), h8(w28)
    w8 = t.empty((2 * N, K), dtype=t.uint8, device="cuda")
    sw.swiglu_pack_fp8(handle, w18, w28, w8, K, N)
    y = t.full((M, N), -1, dtype=t.int16, device="cuda")

    scales = (1.0, 2.0 ** -4, 2.0 ** -4)
    y_ref = oracle.swiglu_fp8_rows(a8_rows, w18_h, w28_h, *scales)
    for variant, cfg in ((sw.VARIANT_INTERLEAVE, 43), (sw.VARIANT_AUTO, -1), (sw.VARIANT_SYNC, 53),
                         (sw.VARIANT_SYNC, -1)):
        y.fill_(-1)
        sw.swiglu_forward_fp8(handle, a8, w8, y, M, N, K, *scales, config_id=cfg, variant=variant)
        t.cuda.synchronize()
        assert_parity(host(y)[rows], y_ref, f"fp8 limit variant {variant} config {cfg}")

    # MXFP8: E8M0 scales around 2^-4 on both sides
    ks = sw.mx_scale_stride(K)
    sa = t.randint(119, 127, (M, ks), device="cuda", generator=g, dtype=t.uint8)
    swt = t.randint(119, 127, (2 * N, ks), device="cuda", generator=g, dtype=t.uint8)
    y_ref = oracle.swiglu_mx_rows(a8_rows, h8(sa[t.from_numpy(rows).cuda()]), h8(w8), h8(swt))
    for cfg in (56, 82):
        y.fill_(-1)
        sw.swiglu_forward_mx(handle, a8, sa, w8, swt, y, M, N, K, ks, config_id=cfg)
        t.cuda.synchronize()
        assert_parity(host(y)[rows], y_ref, f"mx limit config {cfg}")
    del a8, sa, y
