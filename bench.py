#!/usr/bin/env python3
"""Benchmark of the fused SwiGLU MLP GEMM on one MI355X.

One step = one fused forward Y = SiLU(A W1) (.) (A W2) over one batch of the
chosen Qwen2.5-shaped workload (default: the Qwen2.5-72B MLP, M=4096, K=8192,
N=29568, the largest of the five and the MFMA-bound regime), inputs already
resident in HBM.  Batches rotate through enough copies
of {A, W, Y} to exceed the 256 MB Infinity Cache several times, so every step
streams its operands from HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--layout L]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
METRIC = "fused SwiGLU GEMM TFLOP/s (bf16) and % MFMA peak, Qwen2.5-shaped MLPs"
KERNEL_SRC = os.path.join(ROOT, "gemm_epilogues_mlp_amd", "csrc", "swiglu_kernels.hip")


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def _workloads():
    from gemm_epilogues_mlp_amd import inputs as I
    return I.WORKLOADS


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="qwen2.5-72b-mlp",
                   choices=[w.name for w in _workloads()])
    p.add_argument("--layout", choices=["auto", "separate", "interleaved", "packed"],
                   default="auto")
    p.add_argument("--config", type=int, default=-1, help="force a fused config id")
    p.add_argument("--rotate-bytes", type=float, default=1.0 * 2 ** 30,
                   help="minimum footprint of the rotated buffers (bytes)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-unfused", action="store_true")
    p.add_argument("--no-fp8", action="store_true",
                   help="skip the FP8 (E4M3) and MXFP8 side measurements")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 1 GiB device copy (counter calibration runs)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported. The op "
              "needs no collective: under tensor parallelism each GPU runs its own slice of "
              "W_fused columns (cut on Gate/Up pair boundaries) on the full A, so one GPU's "
              "throughput is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import gemm_epilogues_mlp_amd as sw
    from gemm_epilogues_mlp_amd import inputs as I

    wl = I.BY_NAME[args.workload]
    M, K, N = wl.M, wl.K, wl.N
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    h = sw.swiglu_create(0)

    a_np, w1_np, w2_np = I.workload_inputs(wl)
    a0 = torch.from_numpy(a_np.view(np.int16)).to(dev)
    w10 = torch.from_numpy(w1_np.view(np.int16)).to(dev)
    w20 = torch.from_numpy(w2_np.view(np.int16)).to(dev)
    stream = torch.cuda.current_stream()

    if args.layout == "auto":
        _, _, rec = sw.swiglu_query(h, M, N, K, sw.LAYOUT_SEPARATE)
        layout = rec
    else:
        layout = {"interleaved": sw.LAYOUT_INTERLEAVED, "separate": sw.LAYOUT_SEPARATE,
                  "packed": sw.LAYOUT_PACKED}[args.layout]
    variant, tile, _ = sw.swiglu_query(h, M, N, K, layout)
    if args.config >= 0:
        tile = sw.swiglu_config_info(args.config)

    wf0 = None
    if layout == sw.LAYOUT_INTERLEAVED:
        wf0 = torch.empty((K, 2 * N), dtype=torch.int16, device=dev)
        sw.swiglu_pack_interleaved(h, w10, w20, wf0, K, N)
    elif layout == sw.LAYOUT_PACKED:  # fragment-ordered W_fused (offline pack)
        wf0 = torch.empty((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16, device=dev)
        sw.swiglu_pack_fragments(h, w10, w20, wf0, K, N)

    set_bytes = wl.fused_bytes
    nsets = max(1, int(np.ceil(args.rotate_bytes / set_bytes)))
    sets = []
    for i in range(nsets):
        a = a0 if i == 0 else a0.clone()
        if layout in (sw.LAYOUT_INTERLEAVED, sw.LAYOUT_PACKED):
            ws = (wf0 if i == 0 else wf0.clone(), None)
        else:
            ws = (w10 if i == 0 else w10.clone(), w20 if i == 0 else w20.clone())
        y = torch.empty((M, N), dtype=torch.int16, device=dev)
        sets.append((a, ws[0], ws[1], y))
    torch.cuda.synchronize()

    def fused_step(i):
        a, w1, w2, y = sets[i % nsets]
        sw.swiglu_forward_ex(h, a, w1, w2, y, M, N, K, layout, sw.VARIANT_AUTO, args.config,
                             stream)

    def timed(step_fn, steps, warmup, batches=5):
        """ms per step over all `steps` (one span of HIP events on the launch
        stream), plus the per-step time of each of `batches` equal batches."""
        for i in range(warmup):
            step_fn(i)
        torch.cuda.synchronize()
        nb = max(1, min(batches, steps))
        bounds = [round(b * steps / nb) for b in range(nb + 1)]
        events = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
        events[0].record(stream)
        for b in range(nb):
            for i in range(bounds[b], bounds[b + 1]):
                step_fn(warmup + i)
            events[b + 1].record(stream)
        torch.cuda.synchronize()
        per_batch = [events[b].elapsed_time(events[b + 1]) / (bounds[b + 1] - bounds[b])
                     for b in range(nb)]
        return events[0].elapsed_time(events[nb]) / steps, per_batch

    ms, fused_batches = timed(fused_step, args.steps, args.warmup)
    tflops = wl.flops / (ms * 1e-3) / 1e12
    hbm_gbs = wl.fused_bytes / (ms * 1e-3) / 1e9

    # ---- decode on the packed weights with K split over workgroups: a side
    #      measurement (its own entry point, with a caller workspace) ----------
    splitk = None
    if layout == sw.LAYOUT_PACKED and M <= 16 and args.config < 0:
        cfg_k, s_k = sw.swiglu_packed_splitk_plan(h, M, N, K)
        wsk = [torch.zeros((sw.swiglu_packed_splitk_workspace_bytes(N, K, s_k),),
                           dtype=torch.uint8, device=dev) for _ in range(nsets)]

        def splitk_step(i):
            a, w1, _, y = sets[i % nsets]
            sw.swiglu_forward_packed_splitk(h, a, w1, y, M, N, K, wsk[i % nsets], s_k, cfg_k,
                                            stream)

        kms, _ = timed(splitk_step, args.steps, args.warmup)
        splitk = {"ms_per_step": round(kms, 5),
                  "hbm_gbs_algorithmic": round(wl.fused_bytes / (kms * 1e-3) / 1e9, 1),
                  "ksplit": s_k, "tile": sw.swiglu_config_info(cfg_k)}
        del wsk

    # ---- unfused baseline on the same GEMM core (3 launches per step) -------
    unfused = None
    if not args.no_unfused:
        ws_buf = torch.empty((2, M, N), dtype=torch.int16, device=dev)
        usets = []
        if layout == sw.LAYOUT_SEPARATE:
            usets = [(s[0], s[1], s[2], s[3]) for s in sets]
        else:
            usets = [(a0, w10, w20, sets[0][3])]
            for i in range(1, max(1, int(np.ceil(args.rotate_bytes / wl.unfused_bytes)))):
                usets.append((a0.clone(), w10.clone(), w20.clone(),
                              torch.empty((M, N), dtype=torch.int16, device=dev)))

        def unfused_step(i):
            a, w1, w2, y = usets[i % len(usets)]
            sw.swiglu_forward_unfused(h, a, w1, w2, ws_buf, y, M, N, K, -1, stream)

        ums, _ = timed(unfused_step, max(10, args.steps // 2), max(3, args.warmup // 2))
        # fusion efficiency: time saved / time to move the saved bytes at the
        # device-to-device copy rate (1 GiB copy, bytes read + written)
        csrc = torch.empty(2 ** 29, dtype=torch.int16, device=dev)
        cdst = torch.empty_like(csrc)
        cms, _ = timed(lambda i: cdst.copy_(csrc), 10, 3, batches=1)
        copy_gbs = 2 * csrc.numel() * 2 / (cms * 1e-3) / 1e9
        del csrc, cdst
        saved = wl.unfused_bytes - wl.fused_bytes
        unfused = {"ms_per_step": round(ums, 5),
                   "tflops": round(wl.flops / (ums * 1e-3) / 1e12, 2),
                   "fusion_speedup": round(ums / ms, 3),
                   "bytes_saved": saved, "copy_gbs": round(copy_gbs, 1),
                   "fusion_efficiency": round((ums - ms) * 1e-3 / (saved / (copy_gbs * 1e9)), 3),
                   "gemm_tile": sw.swiglu_query_unfused(h, M, N, K)}
        del usets, ws_buf

    # ---- FP8 (E4M3) inputs, per-tensor scales: a side measurement ----------
    fp8 = None
    if not args.no_fp8:
        fp8 = fp8_side(sw, h, wl, a_np, w1_np, w2_np, a0, w10, w20, timed, stream, args, ms)
        fp8["mxfp8"] = mx_side(sw, h, wl, a0, w10, w20, timed, stream, args, ms)

    if args.copy_calibration:
        src = torch.empty(2 ** 30 // 2, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- roofline of the dominant kernel (the fused kernel: 1 launch/step) --
    bound = "mfma" if wl.flops / wl.fused_bytes > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9) \
        else "hbm"
    if bound == "mfma":
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(hbm_gbs / PEAK_HBM_GBS, 4)}
    roofline["traffic"] = counter_traffic(wl.name, layout, tile)

    # ---- CPU baseline: the oracle on a bounded sample of the same workload --
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, a_np, w1_np, w2_np)

    line = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/K) weights)",
        "config": {"workload": wl.name, "M": M, "K": K, "N": N,
                   "layout": {0: "separate", 1: "interleaved", 2: "packed"}[layout],
                   "variant": {sw.VARIANT_INTERLEAVE: "interleave", sw.VARIANT_SYNC: "sync",
                               sw.VARIANT_PACKED: "interleave (fragment-ordered weights)"}[variant],
                   "tile": tile, "rotated_sets": nsets, "parallelism": "single-gpu"},
        "batches": {"n": len(fused_batches),
                    "median_ms_per_step": round(sorted(fused_batches)[len(fused_batches) // 2], 5),
                    "min_ms_per_step": round(min(fused_batches), 5)},
        "env": {"device": torch.cuda.get_device_name(dev),
                "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
                "torch": torch.__version__, "hip": torch.version.hip},
        "pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_gbs_algorithmic": round(hbm_gbs, 1),
        "unfused": unfused,
        "packed_splitk": splitk,
        "fp8": fp8,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    sw.swiglu_destroy(h)
    print(json.dumps(line), flush=True)


def fp8_side(sw, h, wl, a_np, w1_np, w2_np, a0, w10, w20, timed, stream, args, bf16_ms):
    """The same workload on FP8 inputs: A, W1 and W2 quantised on the device
    (scale = max|x| / 448 per tensor), W1 and W2 packed k-major once, then
    the fused FP8 forward timed like the bf16 one.  The per-forward cost of
    quantising bf16 activations is timed separately."""
    import numpy as np
    import torch
    from gemm_epilogues_mlp_amd import inputs as I
    M, K, N = wl.M, wl.K, wl.N
    dev = a0.device

    def scale(bits):
        amax = float(np.max(np.abs(I.bf16_bits_to_f32(bits))))
        return float(np.float32(amax / 448.0)) if amax > 0 else 1.0

    sa, s1, s2 = scale(a_np), scale(w1_np), scale(w2_np)
    a8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    w18 = torch.empty((K, N), dtype=torch.uint8, device=dev)
    w28 = torch.empty_like(w18)
    sw.swiglu_quantize_fp8(h, a0, a8, M * K, 1.0 / sa, stream)
    sw.swiglu_quantize_fp8(h, w10, w18, K * N, 1.0 / s1, stream)
    sw.swiglu_quantize_fp8(h, w20, w28, K * N, 1.0 / s2, stream)
    w8 = torch.empty((2 * N, K), dtype=torch.uint8, device=dev)
    sw.swiglu_pack_fp8(h, w18, w28, w8, K, N, stream)
    del w18, w28
    bytes8 = M * K + 2 * N * K + 2 * M * N
    nsets = max(1, int(np.ceil(args.rotate_bytes / bytes8)))
    sets = [(a8 if i == 0 else a8.clone(), w8 if i == 0 else w8.clone(),
             torch.empty((M, N), dtype=torch.int16, device=dev)) for i in range(nsets)]
    torch.cuda.synchronize()

    def step(i):
        a, w, y = sets[i % nsets]
        sw.swiglu_forward_fp8(h, a, w, y, M, N, K, sa, s1, s2, -1, stream)

    fms, batches = timed(step, args.steps, args.warmup)
    qms, _ = timed(lambda i: sw.swiglu_quantize_fp8(h, a0, a8, M * K, 1.0 / sa, stream),
                   max(10, args.steps // 2), 3, batches=1)
    tf = wl.flops / (fms * 1e-3) / 1e12
    out = {"ms_per_step": round(fms, 5), "tflops": round(tf, 2),
           "pct_fp8_mfma_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
           "speedup_vs_bf16": round(bf16_ms / fms, 3),
           "hbm_gbs_algorithmic": round(bytes8 / (fms * 1e-3) / 1e9, 1),
           "min_batch_ms_per_step": round(min(batches), 5),
           "quantize_activations_ms": round(qms, 5),
           "format": "OCP E4M3, per-tensor fp32 scales", "rotated_sets": nsets,
           "tile": sw.swiglu_query_fp8(h, M, N, K, sw.VARIANT_AUTO)}
    del sets
    if M <= 64:
        # decode-sized batches: the same forward on fragment-ordered W8
        p8 = torch.empty((sw.swiglu_fp8_packed_bytes(N, K),), dtype=torch.uint8, device=dev)
        sw.swiglu_pack_fp8_fragments(h, w8, p8, K, N, stream)
        psets = [(a8 if i == 0 else a8.clone(), p8 if i == 0 else p8.clone(),
                  torch.empty((M, N), dtype=torch.int16, device=dev)) for i in range(nsets)]
        torch.cuda.synchronize()

        def pstep(i):
            a, w, y = psets[i % nsets]
            sw.swiglu_forward_fp8(h, a, w, y, M, N, K, sa, s1, s2, -1, stream,
                                  variant=sw.VARIANT_FP8_PACKED)

        pms, pb = timed(pstep, args.steps, args.warmup)
        out["packed"] = {"ms_per_step": round(pms, 5),
                         "hbm_gbs_algorithmic": round(bytes8 / (pms * 1e-3) / 1e9, 1),
                         "speedup_vs_bf16": round(bf16_ms / pms, 3),
                         "min_batch_ms_per_step": round(min(pb), 5),
                         "tile": sw.swiglu_query_fp8(h, M, N, K, sw.VARIANT_FP8_PACKED)}
        del psets, p8
    del a8, w8
    return out


def mx_side(sw, h, wl, a0, w10, w20, timed, stream, args, bf16_ms):
    """The same workload on MXFP8 inputs (E4M3 elements, an E8M0 scale per 32
    consecutive k): weights paired k-major and quantised once on the device,
    activations quantised on the device (timed separately), then the fused
    MXFP8 forward timed like the bf16 one."""
    import numpy as np
    import torch
    M, K, N = wl.M, wl.K, wl.N
    dev = a0.device
    ks = sw.mx_scale_stride(K)
    wt = torch.empty((2 * N, K), dtype=torch.int16, device=dev)
    sw.swiglu_pack_kmajor(h, w10, w20, wt, K, N, stream)
    qw = torch.empty((2 * N, K), dtype=torch.uint8, device=dev)
    sW = torch.empty((2 * N, ks), dtype=torch.uint8, device=dev)
    sw.swiglu_quantize_mx(h, wt, qw, sW, 2 * N, K, ks, stream)
    del wt
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((M, ks), dtype=torch.uint8, device=dev)
    sw.swiglu_quantize_mx(h, a0, qa, sa, M, K, ks, stream)
    bytes_mx = M * K + 2 * N * K + 2 * M * N + (M + 2 * N) * ks
    nsets = max(1, int(np.ceil(args.rotate_bytes / bytes_mx)))
    sets = [tuple(t if i == 0 else t.clone() for t in (qa, sa, qw, sW)) +
            (torch.empty((M, N), dtype=torch.int16, device=dev),) for i in range(nsets)]
    torch.cuda.synchronize()

    def step(i):
        A8, SA, W8, SW, y = sets[i % nsets]
        sw.swiglu_forward_mx(h, A8, SA, W8, SW, y, M, N, K, ks, -1, stream)

    xms, batches = timed(step, args.steps, args.warmup)
    # the sync (Kernel-1) order on the same W8 and scales
    scfg = sw.swiglu_query_fp8(h, M, N, K, sw.VARIANT_MXFP8_SYNC)

    def sstep(i):
        A8, SA, W8, SW, y = sets[i % nsets]
        sw.swiglu_forward_mx(h, A8, SA, W8, SW, y, M, N, K, ks, scfg["id"], stream)

    sms, _ = timed(sstep, max(10, args.steps // 2), max(3, args.warmup // 2))
    qms, _ = timed(lambda i: sw.swiglu_quantize_mx(h, a0, qa, sa, M, K, ks, stream),
                   max(10, args.steps // 2), 3, batches=1)
    tf = wl.flops / (xms * 1e-3) / 1e12
    out = {"ms_per_step": round(xms, 5), "tflops": round(tf, 2),
           "pct_fp8_mfma_peak": round(100 * tf / PEAK_FP8_TFLOPS, 2),
           "speedup_vs_bf16": round(bf16_ms / xms, 3),
           "min_batch_ms_per_step": round(min(batches), 5),
           "quantize_activations_ms": round(qms, 5),
           "format": "OCP MX: E4M3 elements, E8M0 scale per 32 along K", "rotated_sets": nsets,
           "tile": sw.swiglu_query_fp8(h, M, N, K, sw.VARIANT_MXFP8),
           "sync": {"ms_per_step": round(sms, 5),
                    "tflops": round(wl.flops / (sms * 1e-3) / 1e12, 2), "tile": scfg}}
    del sets
    if M <= 64:
        # decode-sized batches: the same forward on fragment-ordered W8
        p8 = torch.empty((sw.swiglu_mx_packed_bytes(N, K),), dtype=torch.uint8, device=dev)
        sw.swiglu_pack_mx_fragments(h, qw, p8, K, N, stream)
        psets = [tuple(t if i == 0 else t.clone() for t in (qa, sa, p8, sW)) +
                 (torch.empty((M, N), dtype=torch.int16, device=dev),) for i in range(nsets)]
        torch.cuda.synchronize()

        def pstep(i):
            A8, SA, P8, SW, y = psets[i % nsets]
            sw.swiglu_forward_mx_packed(h, A8, SA, P8, SW, y, M, N, K, ks, -1, stream)

        pms, pb = timed(pstep, args.steps, args.warmup)
        out["packed"] = {"ms_per_step": round(pms, 5),
                         "hbm_gbs_algorithmic": round(bytes_mx / (pms * 1e-3) / 1e9, 1),
                         "speedup_vs_bf16": round(bf16_ms / pms, 3),
                         "min_batch_ms_per_step": round(min(pb), 5),
                         "tile": sw.swiglu_query_fp8(h, M, N, K, sw.VARIANT_MXFP8_PACKED)}
        del psets, p8
    del qa, sa, qw, sW
    return out


def counter_traffic(workload, layout, tile):
    """HBM bytes per launch from the committed rocprofv3 counter summary for
    this kernel configuration and workload, if it was taken on the current
    kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    name = {0: "separate", 1: "interleaved", 2: "packed"}.get(layout, str(layout))
    key = f"{workload}/{name}/config{tile.get('id')}"
    entry = data.get(key)
    if not entry or entry.get("kernel_source_sha") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(wl, a, w1, w2):
    """Time the CPU oracle (as it is) on a bounded row sample of the workload."""
    import numpy as np

    import oracle
    nthreads = oracle.default_threads()
    per_row = 4.0 * wl.N * wl.K
    probe = min(wl.M, 8)
    t0 = time.perf_counter()
    oracle.swiglu_rows(a, w1, w2, rows=np.arange(probe), nthreads=nthreads)
    dt = time.perf_counter() - t0
    rate = probe * per_row / max(dt, 1e-9)
    rows = int(min(wl.M, max(probe, 12.0 * rate / per_row)))  # about 12 s of work
    # a sample capped at M rows can take well under the target: repeat whole
    # passes over it until about 10 s have been timed
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.swiglu_rows(a, w1, w2, rows=np.arange(rows), nthreads=nthreads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 1000:
            break
    return {"value": round(passes * rows * per_row / dt / 1e12, 5), "unit": "TFLOP/s",
            "cores": min(nthreads, rows), "kind": "oracle",
            "sample": f"first {rows} of {wl.M} rows of Y (all {wl.N} columns), "
                      f"{passes} pass(es), {dt:.1f} s wall"}


if __name__ == "__main__":
    main()
