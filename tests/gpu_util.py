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
