"""The fused forward captured in a HIP graph (torch.cuda.CUDAGraph over the
C ABI on the capturing stream), replayed several times with eager work and
synchronisations in between: every replay must equal the eager result bit for
bit (same kernels, same configuration).  The kernels issue no memsets, so
nothing in the captured work depends on the first replay."""
import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import assert_parity, dev, host, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


CASES = [  # (M, N, K, layout)
    (16, 4864, 896, sw.LAYOUT_PACKED),
    (128, 4864, 896, sw.LAYOUT_INTERLEAVED),
    (40, 264, 200, sw.LAYOUT_SEPARATE),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}-layout{c[3]}")
def test_graph_replay_equals_eager(handle, case):
    import torch
    M, N, K, layout = case
    a, w1, w2 = I.make_inputs(M, K, N, 21)
    log(f"graph case {case}")
    a_d, w1_d, w2_d = dev(a), dev(w1), dev(w2)
    if layout == sw.LAYOUT_PACKED:
        W1 = torch.empty((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16, device="cuda")
        sw.swiglu_pack_fragments(handle, w1_d, w2_d, W1, K, N)
        W2 = None
    elif layout == sw.LAYOUT_INTERLEAVED:
        W1 = torch.empty((K, 2 * N), dtype=torch.int16, device="cuda")
        sw.swiglu_pack_interleaved(handle, w1_d, w2_d, W1, K, N)
        W2 = None
    else:
        W1, W2 = w1_d, w2_d
    y_eager = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    sw.swiglu_forward(handle, a_d, W1, W2, y_eager, M, N, K, layout)
    torch.cuda.synchronize()
    assert_parity(host(y_eager), oracle.swiglu(a, w1, w2), f"eager {case}")

    y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream once, eagerly
        sw.swiglu_forward(handle, a_d, W1, W2, y, M, N, K, layout)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sw.swiglu_forward(handle, a_d, W1, W2, y, M, N, K, layout)
    for r in range(4):
        y.fill_(-1)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r} differs from the eager forward"
    del g


def test_graph_replay_fp8_fragment_order(handle):
    import torch
    M, N, K = 16, 4864, 896
    rng = np.random.default_rng(5)
    a8 = rng.integers(0, 0x7E, (M, K), dtype=np.uint8)
    w8 = rng.integers(0, 0x7E, (2 * N, K), dtype=np.uint8)
    p8 = torch.from_numpy(oracle.pack_fp8_fragments(w8)).cuda()
    a_d = torch.from_numpy(a8).cuda()
    y_eager = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    sw.swiglu_forward_fp8(handle, a_d, p8, y_eager, M, N, K, 2.0 ** -6, 2.0 ** -9, 2.0 ** -9,
                          variant=sw.VARIANT_FP8_PACKED)
    torch.cuda.synchronize()
    y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sw.swiglu_forward_fp8(handle, a_d, p8, y, M, N, K, 2.0 ** -6, 2.0 ** -9, 2.0 ** -9,
                              variant=sw.VARIANT_FP8_PACKED)
    for r in range(4):
        y.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r} differs from the eager forward"
    del g


def test_graph_replay_splitk(handle):
    """The decode forward with K split over workgroups, captured: its counters
    return to zero in every launch, so every replay runs the handoff afresh on
    the same workspace and equals the eager result bit for bit."""
    import torch
    M, N, K = 9, 1184, 3584
    a, w1, w2 = I.make_inputs(M, K, N, 23)
    a_d, w1_d, w2_d = dev(a), dev(w1), dev(w2)
    P = torch.empty((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16, device="cuda")
    sw.swiglu_pack_fragments(handle, w1_d, w2_d, P, K, N)
    S = 3
    ws = torch.zeros((sw.swiglu_packed_splitk_workspace_bytes(N, K, S),), dtype=torch.uint8,
                     device="cuda")
    y_eager = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    sw.swiglu_forward_packed_splitk(handle, a_d, P, y_eager, M, N, K, ws, ksplit=S)
    torch.cuda.synchronize()
    assert_parity(host(y_eager), oracle.swiglu(a, w1, w2), "split-K eager")
    log(f"graph split-K {(M, N, K)} S={S}")
    y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm the capture stream once, eagerly
        sw.swiglu_forward_packed_splitk(handle, a_d, P, y, M, N, K, ws, ksplit=S)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        sw.swiglu_forward_packed_splitk(handle, a_d, P, y, M, N, K, ws, ksplit=S)
    slabs = (2 * N + 127) // 128
    for r in range(4):
        y.fill_(-1)                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager), f"replay {r} differs from the eager forward"
        assert int(ws[:slabs * 16].count_nonzero().item()) == 0, f"counters after replay {r}"
    del g
