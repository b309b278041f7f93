"""One handle used from several host threads, each enqueueing forwards on a
stream of its own, all at once: the library's contract says a handle holds
host state only and may be shared so.  Every thread's outputs must equal,
bit for bit, what the same calls give run alone on one stream (same kernels,
same configuration), and meet the parity bar against the oracle."""
import threading

import numpy as np
import pytest

import gemm_epilogues_mlp_amd as sw
import oracle
from gemm_epilogues_mlp_amd import inputs as I
from gpu_util import assert_parity, dev, host, log

pytestmark = pytest.mark.gpu

REPEATS = 12

# (M, N, K, entry): the interleaved and separate forwards, the fragment-ordered
# decode forward, and the split-K decode forward with its own workspace
CASES = [
    (200, 1032, 520, "interleaved"),
    (72, 264, 200, "separate"),
    (16, 4864, 896, "packed"),
    (9, 1184, 3584, "splitk"),
]


@pytest.fixture(scope="module")
def handle():
    h = sw.swiglu_create(0)
    yield h
    sw.swiglu_destroy(h)


def _prepare(handle, case, seed):
    import torch
    M, N, K, entry = case
    a, w1, w2 = I.make_inputs(M, K, N, seed)
    a_d, w1_d, w2_d = dev(a), dev(w1), dev(w2)
    c = dict(case=case, ref=oracle.swiglu(a, w1, w2), a=a_d)
    if entry == "interleaved":
        c["w1"] = torch.empty((K, 2 * N), dtype=torch.int16, device="cuda")
        sw.swiglu_pack_interleaved(handle, w1_d, w2_d, c["w1"], K, N)
        c["w2"] = None
    elif entry == "separate":
        c["w1"], c["w2"] = w1_d, w2_d
    else:
        c["w1"] = torch.empty((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16,
                              device="cuda")
        sw.swiglu_pack_fragments(handle, w1_d, w2_d, c["w1"], K, N)
        c["w2"] = None
        if entry == "splitk":
            _, S = sw.swiglu_packed_splitk_plan(handle, M, N, K)
            c["S"] = max(S, 2)  # at least two pieces, so the handoff runs
            c["ws"] = torch.zeros((sw.swiglu_packed_splitk_workspace_bytes(N, K, c["S"]),),
                                  dtype=torch.uint8, device="cuda")
    return c


def _forward(handle, c, y, stream):
    M, N, K, entry = c["case"]
    if entry == "splitk":
        sw.swiglu_forward_packed_splitk(handle, c["a"], c["w1"], y, M, N, K, c["ws"],
                                        ksplit=c["S"], stream=stream)
    else:
        layout = {"interleaved": sw.LAYOUT_INTERLEAVED, "separate": sw.LAYOUT_SEPARATE,
                  "packed": sw.LAYOUT_PACKED}[entry]
        sw.swiglu_forward(handle, c["a"], c["w1"], c["w2"], y, M, N, K, layout, stream=stream)


def test_threads_and_streams_share_a_handle(handle):
    import torch
    cases = [_prepare(handle, case, 900 + i) for i, case in enumerate(CASES)]
    # each case alone, on the current stream
    alone = []
    for c in cases:
        M, N = c["case"][:2]
        y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
        _forward(handle, c, y, None)
        alone.append(y)
    torch.cuda.synchronize()
    for c, y in zip(cases, alone):
        assert_parity(host(y), c["ref"], f"alone {c['case']}")

    # all cases at once: one host thread and one stream each, REPEATS outputs per case
    streams = [torch.cuda.Stream() for _ in cases]
    outs = [[torch.full(c["case"][:2], -1, dtype=torch.int16, device="cuda")
             for _ in range(REPEATS)] for c in cases]
    torch.cuda.synchronize()
    start = threading.Barrier(len(cases))
    errors = []

    def work(i):
        try:
            start.wait()
            with torch.cuda.stream(streams[i]):
                for y in outs[i]:
                    _forward(handle, cases[i], y, streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported by the main thread
            errors.append((i, repr(e)))

    log(f"concurrent forwards: {len(cases)} threads x {REPEATS}")
    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for c, ref_y, ys in zip(cases, alone, outs):
        for r, y in enumerate(ys):
            assert torch.equal(y, ref_y), f"{c['case']}: repeat {r} differs from the lone call"
    split = [c for c in cases if c["case"][3] == "splitk"]
    for c in split:
        slabs = (2 * c["case"][1] + 127) // 128
        assert int(c["ws"][:slabs * 16].count_nonzero().item()) == 0, "split-K counters not reset"
