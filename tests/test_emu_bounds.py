"""CPU bounds emulation of every kernel configuration (no GPU).

The kernel source is compiled for the host against a stand-in device header
(tests/emu/swiglu_device.hpp) with AddressSanitizer, and every workgroup's
threads are run through the real launch functions: each LDS offset, DMA
source, direct global load and (via the sanitizer) global store and LDS
pointer access is checked against the buffers actually allocated.  A kernel
that would touch memory outside its inputs, outputs or LDS fails here instead
of faulting a GPU.  The same runs check LDS ordering (tests/emu/emu_race.cpp):
every LDS access must be separated by the barriers and DMA waits from any
DMA or other wave's access that could land on the same bytes meanwhile.
Data values are not checked (the threads run one after another); parity is
the GPU tests' job.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "emu"))
import build as emu_build  # noqa: E402


@pytest.fixture(scope="module")
def emu(tmp_path_factory):
    if emu_build.clangxx() is None:
        pytest.skip("no host clang++")
    return emu_build.build(str(tmp_path_factory.mktemp("emu")))


def _run(exe, *args, timeout=600):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, timeout=timeout,
                       env=env)
    return r.returncode, r.stdout + r.stderr


# Every emulation run is its own process, so the module starts them all at
# once (the test functions below only collect their results): the small
# launches on up to 8 host threads, the runs with tensors near 2 GiB (a few GiB
# of host memory each) two at a time.
_SMALL_WORKERS = max(1, min(8, os.cpu_count() or 1))
_LARGE_WORKERS = 2


@pytest.fixture(scope="module")
def runs(emu):
    small = cf.ThreadPoolExecutor(_SMALL_WORKERS)
    large = cf.ThreadPoolExecutor(_LARGE_WORKERS)
    futs = {}
    for args in _small_jobs():
        futs[args] = small.submit(_run, emu, *args)
    for args in _large_jobs():
        futs[args] = large.submit(_run, emu, *args, timeout=900)

    def result(*args):
        args = tuple(map(str, args))
        return futs[args].result() if args in futs else _run(emu, *args)

    yield result
    for ex in (small, large):
        ex.shutdown(wait=False, cancel_futures=True)


def test_all_configs_on_the_parity_shapes(runs):
    rc, out = runs()
    assert rc == 0 and "errors: 0" in out, out[-4000:]
    assert out.count(": ok") >= 5 * 40  # every config ran on every shape


# The LDS ordering check (tests/emu/emu_race.cpp) against mistakes planted in
# the emulation's copy of the kernels (tests/emu/build.py): a K-loop wait one
# step short (bf16 and FP8 tiles), an epilogue that reuses the stage ring
# without the barrier that ends the K loop, a persistent kernel that does not
# drain its last loads, an MX K loop that reads a scale group's bytes while
# their DMA may still be in flight, a pair tile whose Up waves read the Gate
# waves' hand-over without the barrier between them.
PLANTED = [
    (1, 40, 128, "LDS read while a DMA into it may land"),
    (1, 42, 128, "LDS read while a DMA into it may land"),
    (2, 40, 128, "LDS accesses of two waves between the same barriers"),
    (2, 43, 128, "LDS write while a DMA into it may land"),
    (3, 36, 128, "DMA still in flight when its thread ends"),
    (4, 56, 1088, "LDS read while a DMA into it may land"),
    (4, 82, 1088, "LDS read while a DMA into it may land"),
    (5, 43, 1088, "LDS read while a DMA into it may land"),
    (1, 89, 128, "LDS read while a DMA into it may land"),
    (2, 89, 128, "LDS accesses of two waves between the same barriers"),
    (6, 89, 128, "LDS accesses of two waves between the same barriers"),
]
# the plants of the FP8 tile's K loop run on a smaller launch with 17 K steps
# (two scale groups of 8 and a short last one)
PLANT_SHAPE = {128: (2048, 8960, 128), 1088: (2008, 4216, 1088)}


@pytest.mark.parametrize("plant,cfg,K,message", PLANTED)
def test_lds_ordering_check_catches_planted_mistakes(runs, plant, cfg, K, message):
    # the same launch without the plant is one of the workload cases below
    rc, out = runs(*_plant_args(plant, cfg, K))
    assert rc != 0 and message in out, out[-4000:]


# (M, N, K, configs): launches whose tile counts exercise the split tail
# (whole rounds of 256-row tiles plus a short last round), the table's
# choices at the workloads' M and N, and decode-sized streaming
CASES = [
    (2008, 4216, 72, [40, 42]),        # 264 tiles: 256 big + 8 split
    (2008, 8440, 72, [41]),            # the same for the 256-column GEMM tiles
    (2048, 8960, 40, [40, 41, 42, 89]),  # 1.5B M and N: 512 big + 48 split
    # the pair tiles (sync family on W1, W2 as stored): split tail at the
    # 1.5B shape above, ragged edges, the smaller tiles at mid and small M
    (2008, 4216, 72, [89, 90, 91, 92]),
    (512, 18944, 64, [90, 91]),
    (128, 4864, 40, [92]),
    (4096, 29568, 40, [89]),           # 72B M and N: whole rounds, no split
    (2008, 4216, 1088, [43, 56, 82]),  # FP8, MX and MX sync split tiles: 17 steps, 3 scale groups a phase
    # the persistent tiles: whole rings of K (K = 128, 256), two or more tiles
    # per workgroup, with and without a quarter-tile last round, ragged M and N
    (2048, 8960, 128, [36, 40, 42, 43, 89]),  # 560 tiles: 2 per workgroup + 48 as quarters
    (4000, 8440, 256, [37]),           # 528 GEMM tiles: + 16 as quarters, ragged M and N
    (4000, 9000, 128, [36]),           # 1136 tiles: a last round of 112, not split
    (4000, 9400, 128, [37]),           # 592 GEMM tiles: a last round of 80, not split
    (2048, 8960, 72, [36]),            # K not a whole ring: the split-tail launch
    (128, 4864, 40, [3, 29, 30]),      # 0.5B M and N
    (16, 18944, 64, [23, 12, 18]),     # 7B decode M and N
    # the table's choices at one GPU's share under 8-way tensor parallelism
    (2048, 1120, 1536, [1, 8]),
    (8192, 2368, 96, [8, 40, 41]),
    (16, 2368, 3584, [27, 30, 64, 11]),
    (128, 608, 896, [5, 12, 67, 30]),
    (4096, 3696, 64, [40, 42, 41]),
    (2048, 1120, 1536, [45, 57, 54]),
    (16, 2368, 3584, [51, 72, 81]),
    # mid-size batches on the 7B and 72B matrices (wide N)
    (128, 18944, 64, [35, 45, 56]),
    (256, 18944, 64, [21, 44]),
    (128, 29568, 64, [31, 45, 56]),
    (32, 29568, 64, [1, 50, 62]),
    (64, 18944, 64, [35, 8, 16, 54]),
    (256, 18944, 64, [39, 15, 53]),
    (512, 18944, 64, [22, 42]),
    (32, 18944, 64, [1, 8, 16]),
    # decode-sized batches on the 0.5B and 1.5B matrices
    (32, 8960, 1536, [27, 30, 46, 75]),
    (64, 4864, 896, [3, 12, 30, 69, 75]),
    (2048, 8960, 1536, [75]),
    (192, 18944, 64, [42, 15, 44, 35]),
    (384, 18944, 64, [8, 45, 22, 40]),
    (768, 18944, 64, [14, 40, 42, 43]),
    (2048, 29568, 64, [44]),
    # FP8 / MXFP8 (K a multiple of 64): split-tail tiles at 1.5B M and N in
    # both orders and with block scales, the small-M tiles and the streaming
    # kernel at the 0.5B and decode shapes
    (2048, 8960, 576, [43, 53, 56]),
    (2008, 4216, 128, [43, 53, 56]),   # whole rounds plus a short split round
    (128, 4864, 896, [46, 55, 57]),
    (16, 18944, 3584, [52, 57]),
    # fragment-ordered weights: decode, 0.5B and ragged shapes for every
    # packed config (odd and even step counts per wave)
    (16, 18944, 3584, list(range(58, 70)) + [88]),  # 88: 256 whole and 160 quarter slabs
    (128, 4864, 896, list(range(58, 70)) + [88]),
    (33, 72, 40, list(range(58, 70)) + [88]),
    (13, 16504, 72, [88]),             # 258 slabs, the last partial: 256 whole, then quarters
    # FP8 on fragment-ordered W8: decode, 0.5B, ragged (partial step of 128)
    (16, 18944, 3584, list(range(70, 77))),
    (128, 4864, 896, list(range(70, 77))),
    (33, 72, 144, list(range(70, 77))),
    # fragment-ordered W_fused with K split over workgroups (3 pieces): a
    # narrow N (one GPU's share under 8-way tensor parallelism), 7B decode
    (16, 2368, 3584, [85, 86, 87]),
    (16, 18944, 3584, [86]),
    # MXFP8 on fragment-ordered W8: decode, 0.5B, ragged row blocks and groups
    (16, 18944, 3584, [77, 78, 79, 80, 81]),
    (128, 4864, 896, [77, 78, 79, 80, 81]),
    (16, 2368, 3584, [80, 81]),
    (33, 72, 1088, [77, 78, 79, 80, 81]),
]


# the LDS ordering check runs on the last workgroups of each launch (the
# ragged edges, the split tail's quarter tiles, the persistent workgroups'
# last tiles); the bounds checks on every workgroup
RACE_BLOCKS = 24


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}")
def test_table_configs_at_workload_sizes(runs, case):
    M, N, K, cfgs = case
    for cfg in cfgs:
        rc, out = runs(*_case_args(M, N, K, cfg))
        assert rc == 0 and "errors: 0" in out, out[-4000:]


# the split-K streaming configs with other numbers of pieces of K: one (no
# handoff), two, more pieces than a shape has K steps (empty pieces)
@pytest.mark.parametrize("ksplit", [1, 2, 7, 64])  # SPLITK_PIECES
def test_splitk_pieces(runs, ksplit):
    for shape in SPLITK_SHAPES:
        for cfg in SPLITK_CONFIGS:
            rc, out = runs(*_splitk_args(ksplit, shape, cfg))
            assert rc == 0 and "errors: 0" in out, out[-4000:]


# tensors just under the 2 GiB limit (largest byte offsets the kernels form):
# A = 2 * 65536 * 16376 B, and W_fused = 4 * 16376 * 32768 B (bf16), and the
# byte tensors of the FP8 kernels; only the last workgroups of each launch are
# emulated (they touch the largest offsets), bounds only (the LDS ordering
# does not depend on the tensor sizes)
LIMIT_CASES = [
    (65536, 64, 16376, [40, 42, 41], 4),
    # the persistent tiles (K a whole number of rings: 2 * 65536 * 16256 B of A)
    (65536, 512, 16256, [36, 37], 4),
    (16, 32768, 16376, [4, 11, 18, 23, 12], 8),
    # fragment-ordered W_fused just under 2 GiB: 511 slabs x 512 steps x 8 KB
    (16, 32704, 16376, list(range(58, 70)) + [85, 86, 87, 88], 8),
    # fragment-ordered W8 just under 2 GiB: 4096 row blocks x 255 steps x 2 KB
    (16, 32768, 32640, list(range(70, 77)), 8),
    # MX fragment-ordered W8 just under 2 GiB: 2048 row blocks x 511 steps x 2 KB
    (16, 32768, 32704, [77, 78, 79, 80, 81], 8),
    (256, 32768, 16376, [1, 8, 16], 4),
    # byte tensors: A8 = 65536 x 32704 B, W8 = 2 x 32768 x 32704 B (K % 64 == 0)
    (65536, 64, 32704, [43, 53, 56, 82], 4),
    (16, 32768, 32704, [47, 52, 55, 57], 8),
]


@pytest.mark.parametrize("case", LIMIT_CASES, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}")
def test_tensors_just_under_2gib(runs, case):
    M, N, K, cfgs, last = case
    for cfg in cfgs:
        rc, out = runs(*_limit_args(M, N, K, cfg, last))
        assert rc == 0 and "errors: 0" in out, out[-4000:]


SPLITK_PIECES = [1, 2, 7, 64]
SPLITK_SHAPES = ((13, 264, 200), (16, 2368, 3584), (1, 8, 8))
SPLITK_CONFIGS = (85, 86, 87)


# command lines of the emulation driver, one per run
def _plant_args(plant, cfg, K):
    return tuple(map(str, ("--plant", plant, "--race-blocks", 8, "--shape", *PLANT_SHAPE[K],
                           cfg)))


def _case_args(M, N, K, cfg):
    return tuple(map(str, ("--race-blocks", RACE_BLOCKS, "--shape", M, N, K, cfg)))


def _splitk_args(ksplit, shape, cfg):
    return tuple(map(str, ("--ksplit", ksplit, "--race-blocks", RACE_BLOCKS, "--shape", *shape,
                           cfg)))


def _limit_args(M, N, K, cfg, last):
    return tuple(map(str, ("--no-races", "--last-blocks", last, "--shape", M, N, K, cfg)))


def _small_jobs():
    jobs = [()]
    jobs += [_plant_args(p, c, K) for p, c, K, _ in PLANTED]
    jobs += [_case_args(M, N, K, c) for M, N, K, cfgs in CASES for c in cfgs]
    jobs += [_splitk_args(k, s, c) for k in SPLITK_PIECES for s in SPLITK_SHAPES
             for c in SPLITK_CONFIGS]
    return jobs


def _large_jobs():
    return [_limit_args(M, N, K, c, last) for M, N, K, cfgs, last in LIMIT_CASES for c in cfgs]
