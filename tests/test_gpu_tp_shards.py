"""GPU parity at one GPU's share of the Qwen2.5-shaped MLPs under 8-way tensor
parallelism (W_fused columns split eight ways on Gate/Up pair boundaries:
[M, N/8, K]), in the configuration the table picks for each layout, and the
unfused baseline.  Inputs follow the workloads' recipe (A ~ N(0, 1),
W ~ N(0, 1/K), seeded, bf16); sampled rows (every column) are checked against
the oracle, the whole Y for unwritten or non-finite elements."""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import assert_parity, decode, dev, empty_poisoned, host, log

pytestmark = pytest.mark.gpu

# (M, K, N): 72B, 7B prefill, 1.5B, 0.5B and 7B decode shares
SHARDS = [(4096, 8192, 3696), (8192, 3584, 2368), (2048, 1536, 1120), (128, 896, 608),
          (16, 3584, 2368)]


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


@pytest.fixture(scope="module", params=SHARDS, ids=lambda s: "x".join(map(str, s)))
def shard(request):
    M, K, N = request.param
    a, w1, w2 = I.make_inputs(M, K, N, 40 + SHARDS.index(request.param))
    rows = np.unique(np.r_[0, 1, M // 2, M - 1, np.random.default_rng(M + N).integers(0, M, 4)])
    y_ref = oracle.swiglu_rows(a, w1, w2, rows=rows)
    return dict(M=M, K=K, N=N, a=a, w1=w1, w2=w2, rows=rows, y_ref=y_ref)


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
    assert_parity(host(y)[d["rows"]], oracle.gate(oracle.decode_bf16(g), oracle.decode_bf16(u)),
                  f"shard {(M, K, N)} unfused")
