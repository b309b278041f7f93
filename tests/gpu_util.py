"""Helpers shared by the GPU tests: device transfer, calls through the C ABI,
and the element-wise parity check.

Parity bar (every output element):  |y - y_ref| <= 0.01 * |y_ref| + 2^-10,
with y the decoded bf16 GPU output and y_ref the oracle's unrounded fp32
value.  The 1 % relative part is the accuracy criterion of "Riepilogo
Tecnico: Sovrapposizione delle Attivazioni a Livello di Tile..." (§Contributi
Chiave, item 3: share of elements with relative error above 1 % against an
FP32 reference); the absolute floor 2^-10 covers outputs near zero.
"""
import sys

import numpy as np

import gemm_epilogues_mlp_amd as sw
from gemm_epilogues_mlp_amd import inputs as I

REL_TOL = 0.01
ABS_TOL = 2.0 ** -10


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch():
    import torch as t
    return t


def dev(bits):
    """uint16 bf16 bit array -> int16 CUDA tensor holding the same bits."""
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def host(tensor):
    return tensor.cpu().numpy().view(np.uint16)


def empty_poisoned(shape):
    """Output buffer filled with bf16 NaN (0xFFFF) so unwritten elements show."""
    t = torch()
    return t.full(shape, -1, dtype=t.int16, device="cuda")


def decode(bits):
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def violations(y_bits, y_ref):
    """Boolean mask of elements outside the parity bar (NaN counts as outside)."""
    y = decode(y_bits)
    ref = np.asarray(y_ref, dtype=np.float64)
    bad = ~(np.abs(y - ref) <= REL_TOL * np.abs(ref) + ABS_TOL)
    return bad


def assert_parity(y_bits, y_ref, what=""):
    bad = violations(y_bits, y_ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        y = decode(y_bits)
        det = ", ".join(f"{tuple(i)}: gpu={y[tuple(i)]!r} ref={float(y_ref[tuple(i)])!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside "
                             f"tolerance; first: {det}")


def rel_err_share(y_bits, y_ref, thresh=0.01):
    """Share of elements whose relative error exceeds `thresh` (elements with
    |y_ref| below 2^-10 are judged on absolute error)."""
    y = decode(y_bits)
    ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y - ref)
    bad = err > thresh * np.maximum(np.abs(ref), ABS_TOL / thresh)
    return float(bad.mean()) if bad.size else 0.0


class Run:
    """One handle plus tensors on the device; forward calls through the C ABI."""

    def __init__(self, handle):
        self.h = handle

    def fused(self, a_d, w1_d, w2_d, M, N, K, layout, config_id=-1, variant=sw.VARIANT_AUTO,
              y=None):
        t = torch()
        y = empty_poisoned((M, N)) if y is None else y
        sw.swiglu_forward_ex(self.h, a_d, w1_d, w2_d, y, M, N, K, layout, variant, config_id)
        t.cuda.synchronize()
        return y

    def unfused(self, a_d, w1_d, w2_d, M, N, K, config_id=-1):
        t = torch()
        ws = t.full((2, M, N), -1, dtype=t.int16, device="cuda")
        y = empty_poisoned((M, N))
        sw.swiglu_forward_unfused(self.h, a_d, w1_d, w2_d, ws, y, M, N, K, config_id)
        t.cuda.synchronize()
        return y, ws[0], ws[1]


def configs_of(variant):
    return [i for i in range(sw.swiglu_config_count())
            if sw.swiglu_config_info(i)["variant"] == variant]


# ---------------------------------------------------------------- whole-output checks
# The full-size checks compare every one of the M x N outputs with the oracle.
# The arithmetic of the check is plain element-wise work on the host (torch's
# CPU kernels, float64, in row chunks to bound memory); nothing of it runs on
# the device that produced the output.

def _t():
    import torch as t
    return t


def _decode64(bits):
    """uint16 bf16 bit array -> torch float64 tensor (exact)."""
    t = _t()
    b = t.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return (b.to(t.int32) << 16).view(t.float32).to(t.float64)


def _chunks(M, N, elems=1 << 24):
    step = max(1, elems // max(N, 1))
    for r0 in range(0, M, step):
        yield r0, min(M, r0 + step)


def full_check(y_bits, y_ref, what=""):
    """Assert the parity bar on EVERY element of y_bits [M, N] against the
    oracle's fp32 y_ref [M, N].  Returns a summary dict: elements checked, the
    page's statistic (share of elements more than 1 % off, with the absolute
    floor below 2^-10), and the worst error as a fraction of its allowance."""
    t = _t()
    y_bits = np.asarray(y_bits)
    y_ref = np.asarray(y_ref)
    assert y_bits.shape == y_ref.shape, (y_bits.shape, y_ref.shape)
    M, N = y_bits.shape
    nbad, nrel, worst, first = 0, 0, 0.0, None
    for r0, r1 in _chunks(M, N):
        y = _decode64(y_bits[r0:r1])
        ref = t.from_numpy(np.ascontiguousarray(y_ref[r0:r1])).to(t.float64)
        err = (y - ref).abs()
        allow = REL_TOL * ref.abs() + ABS_TOL
        bad = ~(err <= allow)                       # NaN counts as outside
        nb = int(bad.sum())
        if nb and first is None:
            idx = t.nonzero(bad)[:5]
            first = ", ".join(f"({int(i[0]) + r0}, {int(i[1])}): gpu={float(y[i[0], i[1]])!r} "
                              f"ref={float(ref[i[0], i[1]])!r}" for i in idx)
        nbad += nb
        nrel += int((err > REL_TOL * t.clamp(ref.abs(), min=ABS_TOL / REL_TOL)).sum())
        ratio = t.nan_to_num(err / allow, nan=float("inf"))
        worst = max(worst, float(ratio.max())) if ratio.numel() else worst
    if nbad:
        raise AssertionError(f"{what}: {nbad} of {M * N} elements outside tolerance; "
                             f"first: {first}")
    return {"elements": M * N, "rel_gt_1pct": nrel / max(1, M * N), "worst_frac": worst}


def rounding_check(x_bits, x_ref, K, what):
    """A bf16 tensor that an unfused pipeline stored (Gate or Up): every
    element must be the round-to-nearest-even of SOME fp32 sum that lies
    within delta = 2^-20 sqrt(K) of the oracle's value x_ref, i.e. a bf16
    value between RNE(x_ref - delta) and RNE(x_ref + delta).  delta bounds
    the difference that the summation order alone makes between two fp32
    dot products of K bf16 products of this magnitude (each add rounds by at
    most half an ulp of a partial sum of order 1; about 14 standard
    deviations of their random walk), so away from rounding midpoints and
    from zero this is RNE(x_ref) itself.  Returns the number of elements that
    differ from RNE(x_ref)."""
    import oracle
    x_bits = np.asarray(x_bits)
    M, N = x_bits.shape
    delta = 2.0 ** -20 * np.sqrt(max(K, 1))
    flips = 0
    for r0, r1 in _chunks(M, N, 1 << 22):
        ref = np.ascontiguousarray(x_ref[r0:r1]).astype(np.float64)
        got = x_bits[r0:r1]
        v = I.bf16_bits_to_f32(got).astype(np.float64)
        lo = I.bf16_bits_to_f32(oracle.round_bf16((ref - delta).astype(np.float32)))
        hi = I.bf16_bits_to_f32(oracle.round_bf16((ref + delta).astype(np.float32)))
        ok = (v >= lo) & (v <= hi)
        if not ok.all():
            i = tuple(np.argwhere(~ok)[0])
            raise AssertionError(
                f"{what}: element ({i[0] + r0}, {i[1]}) stored {int(got[i]):#06x} = {v[i]!r}; "
                f"the oracle's {ref[i]!r} +- {delta:.2e} rounds to [{lo[i]!r}, {hi[i]!r}]")
        flips += int((got != oracle.round_bf16(ref.astype(np.float32))).sum())
    return flips
