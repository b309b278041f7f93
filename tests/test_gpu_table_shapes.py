"""GPU parity at shapes beyond the five workloads that the tuner measured, in
the configuration a handle with the package's shipped tuned file picks for
each layout and input format (the tuned entry where there is one, the
built-in fallback elsewhere), and the unfused baseline:

* one GPU's share of the Qwen2.5-shaped MLPs under 8-way tensor parallelism
  (W_fused columns split eight ways on Gate/Up pair boundaries: [M, N/8, K]);
* mid-size batches (M = 32 ... 1024) on the 7B, 32B and 72B matrices, and on the
  1.5B, 3B and 14B ones (Qwen2.5-3B: K = 2048, N = 11008; 14B: K = 5120,
  N = 13824).

Inputs follow the workloads' recipe (A ~ N(0, 1), W ~ N(0, 1/K), seeded,
bf16); sampled rows (every column) are checked against the oracle, the whole
Y for unwritten or non-finite elements."""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import assert_parity, decode, dev, empty_poisoned, host, log, rounding_check

pytestmark = pytest.mark.gpu

# (M, K, N): 72B, 7B prefill, 1.5B, 0.5B and 7B decode shares; then mid-size
# batches on the 72B, 32B, 7B, 1.5B, 3B and 14B matrices
SHARDS = [(4096, 8192, 3696), (8192, 3584, 2368), (2048, 1536, 1120), (128, 896, 608),
          (16, 3584, 2368),
          (32, 8192, 29568), (64, 8192, 29568), (128, 8192, 29568), (128, 3584, 18944),
          (256, 3584, 18944), (64, 3584, 18944), (512, 3584, 18944), (32, 3584, 18944),
          (1024, 3584, 18944), (32, 1536, 8960), (64, 896, 4864), (192, 3584, 18944),
          (384, 3584, 18944), (768, 3584, 18944), (320, 3584, 18944),
          (96, 1536, 8960), (160, 2048, 11008), (768, 1536, 8960), (96, 896, 4864),
          (96, 3584, 2368), (192, 5120, 13824), (384, 5120, 13824), (128, 5120, 27648),
          (384, 5120, 27648), (128, 8192, 7392), (384, 8192, 7392), (128, 8192, 3696)]


@pytest.fixture(scope="module")
def handle():
    # these shapes take the package's shipped tuned configurations where the
    # tuner measured one, the built-in fallback elsewhere
    h = sw.swiglu_create_tuned(0, sw.TUNED_MI355X)
    yield h
    sw.swiglu_destroy(h)


@pytest.fixture(scope="module", params=SHARDS, ids=lambda s: "x".join(map(str, s)))
def shard(request):
    M, K, N = request.param
    a, w1, w2 = I.make_inputs(M, K, N, 40 + SHARDS.index(request.param))
    rows = np.unique(np.r_[0, 1, M // 2, M - 1, np.random.default_rng(M + N).integers(0, M, 4)])
    y_ref, g_ref, u_ref = oracle.swiglu_rows(a, w1, w2, rows=rows, with_gate_up=True)
    return dict(M=M, K=K, N=N, a=a, w1=w1, w2=w2, rows=rows, y_ref=y_ref, g_ref=g_ref,
                u_ref=u_ref)


@pytest.mark.parametrize("layout", [sw.LAYOUT_INTERLEAVED, sw.LAYOUT_SEPARATE, sw.LAYOUT_PACKED],
                         ids=["interleaved", "separate", "packed"])
def test_shard_parity(handle, shard, layout):
    import torch
    d = shard
    M, K, N = d["M"], d["K"], d["N"]
    v, tile, _ = sw.swiglu_query(handle, M, N, K, layout)
    log(f"shard {(M, K, N)} layout {layout} -> config {tile['id']}")
    a, w1, w2 = dev(d["a"]), dev(d["w1"]), dev(d["w2"])
    if layout == sw.LAYOUT_INTERLEAVED:
        W1 = torch.empty((K, 2 * N), dtype=torch.int16, device="cuda")
        sw.swiglu_pack_interleaved(handle, w1, w2, W1, K, N)
        W2 = None
    elif layout == sw.LAYOUT_PACKED:
        W1 = torch.empty((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16, device="cuda")
        sw.swiglu_pack_fragments(handle, w1, w2, W1, K, N)
        W2 = None
    else:
        W1, W2 = w1, w2
    y = empty_poisoned((M, N))
    sw.swiglu_forward(handle, a, W1, W2, y, M, N, K, layout)
    torch.cuda.synchronize()
    yb = host(y)
    assert np.all(np.isfinite(decode(yb))), "unwritten or non-finite outputs"
    assert_parity(yb[d["rows"]], d["y_ref"], f"shard {(M, K, N)} layout {layout}")


def test_shard_unfused(handle, shard):
    import torch
    d = shard
    M, K, N = d["M"], d["K"], d["N"]
    log(f"shard {(M, K, N)} unfused gemm config {sw.swiglu_query_unfused(handle, M, N, K)['id']}")
    ws = torch.empty((2, M, N), dtype=torch.int16, device="cuda")
    y = empty_poisoned((M, N))
    sw.swiglu_forward_unfused(handle, dev(d["a"]), dev(d["w1"]), dev(d["w2"]), ws, y, M, N, K)
    torch.cuda.synchronize()
    g, u = host(ws[0])[d["rows"]], host(ws[1])[d["rows"]]
    # G and U: the bf16 rounding of the oracle's sums (up to summation order),
    # then Y against the oracle's gate on those values
    rounding_check(g, d["g_ref"], K, f"shard {(M, K, N)} unfused G")
    rounding_check(u, d["u_ref"], K, f"shard {(M, K, N)} unfused U")
    assert_parity(host(y)[d["rows"]], oracle.gate(oracle.decode_bf16(g), oracle.decode_bf16(u)),
                  f"shard {(M, K, N)} unfused")


def _e4m3(x):
    """(codes, scale): the oracle's quantiser, scale = max|x| / 448 per tensor."""
    amax = np.float32(np.max(np.abs(x)))
    s = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
    return oracle.quantize_e4m3(x, np.float32(1.0) / s), float(s)


@pytest.mark.parametrize("fmt", ["fp8", "fp8-sync", "fp8-packed", "mxfp8", "mxfp8-packed"])
def test_shard_fp8_parity(handle, shard, fmt):
    """The FP8 (per-tensor E4M3) and MXFP8 forwards at the shard shapes, in
    the table's configuration, against the oracle on the same codes."""
    import torch
    d = shard
    M, K, N = d["M"], d["K"], d["N"]
    rows = d["rows"]
    t8 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    y = empty_poisoned((M, N))
    if fmt.startswith("fp8"):
        if "fp8" not in d:  # quantised once per shape, shared by the FP8 formats
            (a8, sa), (w18, s1), (w28, s2) = (_e4m3(I.bf16_bits_to_f32(x))
                                              for x in (d["a"], d["w1"], d["w2"]))
            d["fp8"] = (a8, sa, w18, s1, w28, s2, oracle.pack_fp8_kmajor(w18, w28))
        a8, sa, w18, s1, w28, s2, w8 = d["fp8"]
        variant = {"fp8": sw.VARIANT_INTERLEAVE, "fp8-sync": sw.VARIANT_SYNC,
                   "fp8-packed": sw.VARIANT_FP8_PACKED}[fmt]
        wt = oracle.pack_fp8_fragments(w8) if fmt == "fp8-packed" else w8
        log(f"shard {(M, K, N)} {fmt} -> config "
            f"{sw.swiglu_query_fp8(handle, M, N, K, variant)['id']}")
        sw.swiglu_forward_fp8(handle, t8(a8), t8(wt), y, M, N, K, sa, s1, s2, variant=variant)
        y_ref = oracle.swiglu_fp8_rows(a8, w18, w28, sa, s1, s2, rows=rows)
    else:
        if "mx" not in d:  # quantised once per shape, shared by the MXFP8 formats
            d["mx"] = oracle.quantize_mx(I.bf16_bits_to_f32(d["a"])) + oracle.quantize_mx(
                I.bf16_bits_to_f32(oracle.pack_kmajor_bf16(d["w1"], d["w2"])))
        qa, sa, qw, sw_ = d["mx"]
        ks = sa.shape[1]
        if fmt == "mxfp8":
            log(f"shard {(M, K, N)} {fmt} -> config "
                f"{sw.swiglu_query_fp8(handle, M, N, K, sw.VARIANT_MXFP8)['id']}")
            sw.swiglu_forward_mx(handle, t8(qa), t8(sa), t8(qw), t8(sw_), y, M, N, K, ks)
        else:
            log(f"shard {(M, K, N)} {fmt} -> config "
                f"{sw.swiglu_query_fp8(handle, M, N, K, sw.VARIANT_MXFP8_PACKED)['id']}")
            sw.swiglu_forward_mx_packed(handle, t8(qa), t8(sa), t8(oracle.pack_mx_fragments(qw)),
                                        t8(sw_), y, M, N, K, ks)
        y_ref = oracle.swiglu_mx_rows(qa, sa, qw, sw_, rows=rows)
    torch.cuda.synchronize()
    yb = host(y)
    assert np.all(np.isfinite(decode(yb))), "unwritten or non-finite outputs"
    assert_parity(yb[rows], y_ref, f"shard {(M, K, N)} {fmt}")
