"""Per-shape tuner: times every compiled configuration of a variant on given
shapes and writes a tuned file that swiglu_create_tuned() applies (format in
include/swiglu.h).

Rule ("additive, never regress"): a shape gets an entry only when its best
configuration beats the built-in table's choice for that shape by more than
`margin`, both timed in the same run on the same inputs; every other shape
keeps the built-in choice.  Entries of an existing file given with --merge
are kept for the shapes not re-tuned.  The file is bound to the list of
compiled configurations by its signature, so it cannot outlive a rebuild
that changes that list.

  python -m gemm_epilogues_mlp_amd.tune --shapes 2048x1536x8960 --out tuned.txt
  (shapes are M x K x N, the order of the workload names; --variants picks
  among interleave, sync, gemm, fp8, fp8-sync and mxfp8)
"""
from __future__ import annotations

import argparse
import datetime
import os
import sys

import gemm_epilogues_mlp_amd as sw

VARIANTS = {"interleave": sw.VARIANT_INTERLEAVE, "sync": sw.VARIANT_SYNC, "gemm": sw.VARIANT_GEMM,
            "fp8": sw.VARIANT_FP8, "fp8-sync": sw.VARIANT_FP8_SYNC, "mxfp8": sw.VARIANT_MXFP8,
            "packed": sw.VARIANT_PACKED, "fp8-packed": sw.VARIANT_FP8_PACKED,
            "mxfp8-packed": sw.VARIANT_MXFP8_PACKED, "mxfp8-sync": sw.VARIANT_MXFP8_SYNC}
# the forward's variant argument for each FP8 configuration family
_FP8_ORDER = {sw.VARIANT_FP8: sw.VARIANT_INTERLEAVE, sw.VARIANT_FP8_SYNC: sw.VARIANT_SYNC,
              sw.VARIANT_MXFP8: sw.VARIANT_MXFP8, sw.VARIANT_FP8_PACKED: sw.VARIANT_FP8_PACKED,
              sw.VARIANT_MXFP8_PACKED: sw.VARIANT_MXFP8_PACKED,
              sw.VARIANT_MXFP8_SYNC: sw.VARIANT_MXFP8_SYNC}


def _candidates(variant, M, configs=None):
    ids = configs if configs is not None else range(sw.swiglu_config_count())
    out = []
    for i in ids:
        c = sw.swiglu_config_info(i)
        if c["variant"] != variant:
            continue
        if c["family"] == 1 and M > 256:  # split-K streaming is for small M only
            continue
        if c["family"] != 1 and M <= 16 and c["bm"] > 64:
            continue
        out.append(i)
    return out


def _time_configs(h, variant, M, N, K, ids, reps, rotate_bytes, seed=0):
    """{config id: microseconds per call} over rotated input sets."""
    import torch

    dev = torch.device("cuda")
    g = torch.Generator(device=dev).manual_seed(seed)

    def rnd(shape, scale=1.0):
        return (torch.randn(shape, device=dev, generator=g) * scale).to(torch.bfloat16).view(
            torch.int16)

    fp8 = variant in _FP8_ORDER
    ks = sw.mx_scale_stride(K)
    per_set = (M * K + 2 * K * N + 2 * M * N + (M + 2 * N) * ks) if fp8 else \
        (2 * M * K + 4 * K * N + 2 * M * N)
    nsets = max(1, min(16, -(-int(rotate_bytes) // max(per_set, 1))))
    sets = []
    for _ in range(nsets):
        if fp8:
            # random finite E4M3 codes and E8M0 scales near 2^-7 (values do not
            # change the timing)
            codes = lambda shape: torch.randint(0, 0x7E, shape, device=dev, generator=g,
                                                dtype=torch.uint8)
            y = torch.empty((M, N), dtype=torch.int16, device=dev)
            wshape = {sw.VARIANT_FP8_PACKED: (sw.swiglu_fp8_packed_bytes(N, K),),
                      sw.VARIANT_MXFP8_PACKED: (sw.swiglu_mx_packed_bytes(N, K),)}.get(
                          variant, (2 * N, K))
            sets.append((codes((M, K)), codes(wshape),
                         torch.full((M, ks), 120, dtype=torch.uint8, device=dev),
                         torch.full((2 * N, ks), 120, dtype=torch.uint8, device=dev), y, None))
            continue
        a = rnd((M, K))
        w1, w2 = rnd((K, N), K ** -0.5), rnd((K, N), K ** -0.5)
        if variant == sw.VARIANT_PACKED:
            wf = torch.empty((sw.swiglu_packed_bytes(N, K) // 2,), dtype=torch.int16, device=dev)
            sw.swiglu_pack_fragments(h, w1, w2, wf, K, N)
        else:
            wf = torch.empty((K, 2 * N), dtype=torch.int16, device=dev)
        if variant == sw.VARIANT_INTERLEAVE:
            sw.swiglu_pack_interleaved(h, w1, w2, wf, K, N)
        y = torch.empty((M, N), dtype=torch.int16, device=dev)
        ws = torch.empty((2, M, N), dtype=torch.int16, device=dev) if variant == sw.VARIANT_GEMM \
            else None
        sets.append((a, w1, w2, wf, y, ws))
    stream = torch.cuda.current_stream()

    def call(i, cid):
        if fp8:
            a8, w8, sa, sw8, y, _ = sets[i % nsets]
            if variant in (sw.VARIANT_MXFP8, sw.VARIANT_MXFP8_SYNC):
                sw.swiglu_forward_mx(h, a8, sa, w8, sw8, y, M, N, K, ks, cid, stream)
            elif variant == sw.VARIANT_MXFP8_PACKED:
                sw.swiglu_forward_mx_packed(h, a8, sa, w8, sw8, y, M, N, K, ks, cid, stream)
            else:
                sw.swiglu_forward_fp8(h, a8, w8, y, M, N, K, config_id=cid, stream=stream,
                                      variant=_FP8_ORDER[variant])
            return
        a, w1, w2, wf, y, ws = sets[i % nsets]
        if variant == sw.VARIANT_INTERLEAVE:
            sw.swiglu_forward_ex(h, a, wf, None, y, M, N, K, sw.LAYOUT_INTERLEAVED, variant, cid,
                                 stream)
        elif variant == sw.VARIANT_PACKED:
            sw.swiglu_forward_ex(h, a, wf, None, y, M, N, K, sw.LAYOUT_PACKED, variant, cid,
                                 stream)
        elif variant == sw.VARIANT_SYNC:
            sw.swiglu_forward_ex(h, a, w1, w2, y, M, N, K, sw.LAYOUT_SEPARATE, variant, cid,
                                 stream)
        else:
            sw.swiglu_forward_unfused(h, a, w1, w2, ws, y, M, N, K, cid, stream)

    times = {}
    for cid in ids:
        try:
            for i in range(3):
                call(i, cid)
        except sw.SwiGLUError:  # configuration cannot take this shape
            continue
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            call(i, cid)
        e1.record(stream)
        torch.cuda.synchronize()
        times[cid] = e0.elapsed_time(e1) * 1e3 / reps
    del sets
    torch.cuda.empty_cache()
    return times


def read_entries(path):
    """Entries of a valid tuned file as {(variant, M, N, K): line}."""
    sw.swiglu_tuned_check(path)  # raises unless its signature matches the loaded library
    out = {}
    header = False
    for line in open(path):
        t = line.strip()
        if not t or t.startswith("#"):
            continue
        if not header:
            header = True
            continue
        v, M, N, K = (int(x) for x in t.split()[:4])
        out[(v, M, N, K)] = t
    return out


def tune(shapes, variants=("interleave", "sync", "gemm"), out=None, merge=None, margin=0.03,
         reps=None, rotate_bytes=512 * 2 ** 20, configs=None, log=print):
    """Tune `shapes` [(M, K, N), ...]; returns {(variant, M, N, K): line} of
    the entries written.  `configs` restricts the candidates (ids)."""
    import torch

    entries = read_entries(merge) if merge else {}
    h = sw.swiglu_create(0)
    try:
        for (M, K, N) in shapes:
            for name in variants:
                v = VARIANTS[name]
                if v == sw.VARIANT_GEMM:
                    builtin = sw.swiglu_query_unfused(h, M, N, K)["id"]
                elif v in _FP8_ORDER:
                    builtin = sw.swiglu_query_fp8(h, M, N, K, _FP8_ORDER[v])["id"]
                else:
                    layout = {sw.VARIANT_INTERLEAVE: sw.LAYOUT_INTERLEAVED,
                              sw.VARIANT_PACKED: sw.LAYOUT_PACKED}.get(v, sw.LAYOUT_SEPARATE)
                    builtin = sw.swiglu_query(h, M, N, K, layout)[1]["id"]
                ids = sorted(set(_candidates(v, M, configs)) | {builtin})
                flops = 4.0 * M * N * K
                n = reps or max(5, min(200, int(2e12 / max(flops, 1.0))))
                t = _time_configs(h, v, M, N, K, ids, n, rotate_bytes)
                best = min(t, key=t.get)
                key = (v, M, N, K)
                gain = 1.0 - t[best] / t[builtin]
                log(f"{name} M={M} K={K} N={N}: built-in config {builtin} {t[builtin]:.1f} us, "
                    f"best config {best} {t[best]:.1f} us ({100 * gain:+.1f} %)")
                if best != builtin and gain > margin:
                    entries[key] = f"{v} {M} {N} {K} {best} {t[best]:.2f}us builtin {builtin} " \
                                   f"{t[builtin]:.2f}us"
                else:
                    entries.pop(key, None)  # the built-in choice stands
    finally:
        sw.swiglu_destroy(h)
    if out:
        arch = torch.cuda.get_device_properties(0).gcnArchName.split(":")[0]
        with open(out, "w") as f:
            f.write(f"# tuned SwiGLU configurations, {datetime.datetime.now():%Y-%m-%d %H:%M}, "
                    f"{torch.cuda.get_device_name(0)}\n")
            f.write(f"swiglu-tuned {sw.swiglu_config_signature():016x} {arch}\n")
            for key in sorted(entries):
                f.write(entries[key] + "\n")
        sw.swiglu_tuned_check(out)
    return entries


def _parse_shapes(text):
    shapes = []
    for item in text.split(","):
        M, K, N = (int(x) for x in item.lower().split("x"))
        shapes.append((M, K, N))
    return shapes


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--shapes", required=True, help="MxKxN[,MxKxN...]")
    p.add_argument("--variants", default="interleave,sync,gemm",
                   help="any of " + ",".join(VARIANTS))
    p.add_argument("--out", required=True)
    p.add_argument("--merge", default=None, help="existing tuned file to extend")
    p.add_argument("--margin", type=float, default=0.03)
    p.add_argument("--reps", type=int, default=None)
    a = p.parse_args(argv)
    tune(_parse_shapes(a.shapes), a.variants.split(","), a.out, a.merge, a.margin, a.reps)
    print(f"wrote {a.out}")


if __name__ == "__main__":
    sys.exit(main())
