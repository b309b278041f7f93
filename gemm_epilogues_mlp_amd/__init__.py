"""Python binding of libswiglu.so, the MI355X fused SwiGLU MLP GEMM library.

Argument marshalling only: every function below has the name of the C entry
point it calls (see include/swiglu.h) and passes device pointers, sizes and
the HIP stream through ctypes.  All arithmetic runs in the library's HIP
kernels; there is no fallback of any kind -- if libswiglu.so is missing or
cannot be loaded the call raises.  PyTorch only provides device memory and
the current stream.

Y = SiLU(A W1) (.) (A W2)  ("Riepilogo Tecnico: Sovrapposizione delle
Attivazioni a Livello di Tile...", §Definizione del Problema).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SwiGLUError", "load", "lib_path", "Handle",
    "swiglu_create", "swiglu_destroy", "swiglu_forward", "swiglu_forward_ex",
    "swiglu_forward_unfused", "swiglu_unfused_workspace_bytes",
    "swiglu_pack_interleaved", "swiglu_query", "swiglu_query_unfused",
    "swiglu_config_count", "swiglu_config_info", "swiglu_status_str",
    "swiglu_config_signature", "swiglu_tuned_check", "swiglu_create_tuned",
    "swiglu_forward_fp8", "swiglu_quantize_fp8", "swiglu_pack_fp8", "swiglu_query_fp8",
    "LAYOUT_SEPARATE", "LAYOUT_INTERLEAVED",
    "VARIANT_AUTO", "VARIANT_SYNC", "VARIANT_INTERLEAVE", "VARIANT_GEMM", "VARIANT_FP8",
    "VARIANT_FP8_SYNC", "VARIANT_MXFP8", "swiglu_forward_mx", "swiglu_quantize_mx",
    "swiglu_pack_kmajor", "LAYOUT_PACKED", "VARIANT_PACKED", "swiglu_packed_bytes",
    "swiglu_pack_fragments", "VARIANT_FP8_PACKED", "swiglu_fp8_packed_bytes",
    "swiglu_pack_fp8_fragments", "VARIANT_MXFP8_PACKED", "swiglu_forward_mx_packed",
    "swiglu_mx_packed_bytes", "swiglu_pack_mx_fragments",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libswiglu.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_DEVICE, ERR_LAUNCH, ERR_ALLOC = range(6)
LAYOUT_SEPARATE, LAYOUT_INTERLEAVED, LAYOUT_PACKED = 0, 1, 2
VARIANT_AUTO, VARIANT_SYNC, VARIANT_INTERLEAVE, VARIANT_GEMM, VARIANT_FP8, VARIANT_FP8_SYNC, \
    VARIANT_MXFP8, VARIANT_PACKED, VARIANT_FP8_PACKED, VARIANT_MXFP8_PACKED, VARIANT_MXFP8_SYNC, \
    VARIANT_PACKED_SPLITK = 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11


class SwiGLUError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {swiglu_status_str(status)} (status {status})")


class Tile(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("id", "variant", "family", "bm", "bn", "bk", "waves", "split_k", "lds_bytes",
                 "tail_split")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libswiglu.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is missing: build it with "
            "`python -m gemm_epilogues_mlp_amd._build` (hipcc, gfx950)")
    try:  # share the HIP runtime torch loaded (same soname), if torch is present
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the C ABI itself needs no torch
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    st = ctypes.c_int
    sig = {
        "swiglu_create": ([ctypes.POINTER(p), ctypes.c_int], st),
        "swiglu_destroy": ([p], st),
        "swiglu_forward": ([p, p, p, p, p, i64, i64, i64, ctypes.c_int, p], st),
        "swiglu_forward_ex": ([p, p, p, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int,
                               i32, p], st),
        "swiglu_unfused_workspace_bytes": ([i64, i64], i64),
        "swiglu_forward_unfused": ([p, p, p, p, p, p, i64, i64, i64, i32, p], st),
        "swiglu_forward_unfused_static": ([p, p, p, p, p, i64, i64, i64, i32, p], st),
        "swiglu_pack_interleaved": ([p, p, p, p, i64, i64, p], st),
        "swiglu_query": ([p, i64, i64, i64, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                          ctypes.POINTER(Tile), ctypes.POINTER(ctypes.c_int)], st),
        "swiglu_query_unfused": ([p, i64, i64, i64, ctypes.POINTER(Tile)], st),
        "swiglu_config_count": ([], i32),
        "swiglu_config_info": ([i32, ctypes.POINTER(Tile)], st),
        "swiglu_status_str": ([ctypes.c_int], ctypes.c_char_p),
        "swiglu_config_signature": ([], ctypes.c_uint64),
        "swiglu_tuned_check": ([ctypes.c_char_p, ctypes.POINTER(i32)], st),
        "swiglu_create_tuned": ([ctypes.POINTER(p), ctypes.c_int, ctypes.c_char_p], st),
        "swiglu_forward_fp8": ([p, p, p, p, i64, i64, i64, ctypes.c_float, ctypes.c_float,
                                ctypes.c_float, ctypes.c_int, i32, p], st),
        "swiglu_quantize_fp8": ([p, p, p, i64, ctypes.c_float, p], st),
        "swiglu_pack_fp8": ([p, p, p, p, i64, i64, p], st),
        "swiglu_query_fp8": ([p, i64, i64, i64, ctypes.c_int, ctypes.POINTER(Tile)], st),
        "swiglu_forward_mx": ([p, p, p, p, p, p, i64, i64, i64, i64, i32, p], st),
        "swiglu_quantize_mx": ([p, p, p, p, i64, i64, i64, p], st),
        "swiglu_pack_kmajor": ([p, p, p, p, i64, i64, p], st),
        "swiglu_packed_bytes": ([i64, i64], i64),
        "swiglu_pack_fragments": ([p, p, p, p, i64, i64, p], st),
        "swiglu_fp8_packed_bytes": ([i64, i64], i64),
        "swiglu_pack_fp8_fragments": ([p, p, p, i64, i64, p], st),
        "swiglu_forward_mx_packed": ([p, p, p, p, p, p, i64, i64, i64, i64, i32, p], st),
        "swiglu_mx_packed_bytes": ([i64, i64], i64),
        "swiglu_pack_mx_fragments": ([p, p, p, i64, i64, p], st),
        "swiglu_packed_splitk_workspace_bytes": ([i64, i64, i32], i64),
        "swiglu_packed_splitk_plan": ([p, i64, i64, i64, ctypes.POINTER(i32),
                                       ctypes.POINTER(i32)], st),
        "swiglu_forward_packed_splitk": ([p, p, p, p, i64, i64, i64, i32, i32, p, i64, p], st),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != OK:
        raise SwiGLUError(status, where)


def _ptr(x) -> int | None:
    """Device pointer of a tensor (data_ptr), an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def swiglu_status_str(status: int) -> str:
    return load().swiglu_status_str(status).decode()


def swiglu_create(device: int = 0) -> int:
    """Returns the opaque handle (an address)."""
    h = ctypes.c_void_p()
    _check(load().swiglu_create(ctypes.byref(h), device), "swiglu_create")
    return h.value


def swiglu_config_signature() -> int:
    return load().swiglu_config_signature()


def swiglu_tuned_check(path: str) -> int:
    """Number of entries of a valid tuned file; raises SwiGLUError otherwise."""
    n = ctypes.c_int32()
    _check(load().swiglu_tuned_check(os.fsencode(path), ctypes.byref(n)), "swiglu_tuned_check")
    return n.value


# Tuned configurations measured on MI355X for shapes beyond the five built-in
# workload entries (tensor-parallel shares, other Qwen2.5 matrices, mid-size
# batches); pass to swiglu_create_tuned.
TUNED_MI355X = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuned_mi355x.txt")


def swiglu_create_tuned(device: int = 0, path: str | None = None) -> int:
    h = ctypes.c_void_p()
    _check(load().swiglu_create_tuned(ctypes.byref(h), device,
                                      os.fsencode(path) if path is not None else None),
           "swiglu_create_tuned")
    return h.value


def swiglu_destroy(handle: int) -> None:
    _check(load().swiglu_destroy(handle), "swiglu_destroy")


def swiglu_forward(handle, A, W1, W2, Y, M, N, K, layout=LAYOUT_SEPARATE, stream=None):
    _check(load().swiglu_forward(handle, _ptr(A), _ptr(W1), _ptr(W2), _ptr(Y), M, N, K,
                                 layout, _stream(stream)), "swiglu_forward")


def swiglu_forward_ex(handle, A, W1, W2, Y, M, N, K, layout, variant=VARIANT_AUTO,
                      config_id=-1, stream=None):
    _check(load().swiglu_forward_ex(handle, _ptr(A), _ptr(W1), _ptr(W2), _ptr(Y), M, N, K,
                                    layout, variant, config_id, _stream(stream)),
           "swiglu_forward_ex")


def swiglu_unfused_workspace_bytes(M: int, N: int) -> int:
    return load().swiglu_unfused_workspace_bytes(M, N)


def swiglu_forward_unfused(handle, A, W1, W2, workspace, Y, M, N, K, gemm_config_id=-1,
                           stream=None):
    _check(load().swiglu_forward_unfused(handle, _ptr(A), _ptr(W1), _ptr(W2), _ptr(workspace),
                                         _ptr(Y), M, N, K, gemm_config_id, _stream(stream)),
           "swiglu_forward_unfused")


def swiglu_forward_unfused_static(handle, A, W1, W2, Y, M, N, K, gemm_config_id=-1,
                                  stream=None):
    _check(load().swiglu_forward_unfused_static(handle, _ptr(A), _ptr(W1), _ptr(W2), _ptr(Y),
                                                M, N, K, gemm_config_id, _stream(stream)),
           "swiglu_forward_unfused_static")


STATIC_SCRATCH_BYTES = 128 * 1024 * 1024  # SWIGLU_STATIC_SCRATCH_BYTES in include/swiglu.h


def swiglu_pack_interleaved(handle, W1, W2, W_fused, K, N, stream=None):
    _check(load().swiglu_pack_interleaved(handle, _ptr(W1), _ptr(W2), _ptr(W_fused), K, N,
                                          _stream(stream)), "swiglu_pack_interleaved")


def swiglu_packed_bytes(N: int, K: int) -> int:
    return int(load().swiglu_packed_bytes(N, K))


def swiglu_pack_fragments(handle, W1, W2, P, K, N, stream=None):
    _check(load().swiglu_pack_fragments(handle, _ptr(W1), _ptr(W2), _ptr(P), K, N,
                                        _stream(stream)), "swiglu_pack_fragments")


def swiglu_fp8_packed_bytes(N: int, K: int) -> int:
    return int(load().swiglu_fp8_packed_bytes(N, K))


def swiglu_pack_fp8_fragments(handle, W8, P8, K, N, stream=None):
    _check(load().swiglu_pack_fp8_fragments(handle, _ptr(W8), _ptr(P8), K, N, _stream(stream)),
           "swiglu_pack_fp8_fragments")


def swiglu_query(handle, M, N, K, layout=LAYOUT_SEPARATE):
    """(chosen variant, tile dict, recommended layout)."""
    v, rl, t = ctypes.c_int(), ctypes.c_int(), Tile()
    _check(load().swiglu_query(handle, M, N, K, layout, ctypes.byref(v), ctypes.byref(t),
                               ctypes.byref(rl)), "swiglu_query")
    return v.value, t.as_dict(), rl.value


def swiglu_query_unfused(handle, M, N, K):
    t = Tile()
    _check(load().swiglu_query_unfused(handle, M, N, K, ctypes.byref(t)), "swiglu_query_unfused")
    return t.as_dict()


def swiglu_forward_fp8(handle, A8, W8, Y, M, N, K, scale_a=1.0, scale_w1=1.0, scale_w2=1.0,
                       config_id=-1, stream=None, variant=VARIANT_AUTO):
    """A8 [M, K] and W8 [2N, K] hold E4M3 codes (uint8 tensors; with variant
    VARIANT_FP8_PACKED, W8 is the fragment-ordered copy); Y bf16 [M, N]."""
    _check(load().swiglu_forward_fp8(handle, _ptr(A8), _ptr(W8), _ptr(Y), M, N, K, scale_a,
                                     scale_w1, scale_w2, variant, config_id, _stream(stream)),
           "swiglu_forward_fp8")


def swiglu_forward_mx(handle, A8, SA, W8, SW, Y, M, N, K, ks, config_id=-1, stream=None):
    """MXFP8: A8 [M, K] + SA [M, ks], W8 [2N, K] + SW [2N, ks] (uint8); Y bf16 [M, N]."""
    _check(load().swiglu_forward_mx(handle, _ptr(A8), _ptr(SA), _ptr(W8), _ptr(SW), _ptr(Y), M,
                                    N, K, ks, config_id, _stream(stream)), "swiglu_forward_mx")


def swiglu_forward_mx_packed(handle, A8, SA, P8, SW, Y, M, N, K, ks, config_id=-1,
                             stream=None):
    _check(load().swiglu_forward_mx_packed(handle, _ptr(A8), _ptr(SA), _ptr(P8), _ptr(SW),
                                           _ptr(Y), M, N, K, ks, config_id, _stream(stream)),
           "swiglu_forward_mx_packed")


def swiglu_packed_splitk_workspace_bytes(N: int, K: int, ksplit: int) -> int:
    return int(load().swiglu_packed_splitk_workspace_bytes(N, K, ksplit))


def swiglu_packed_splitk_plan(handle, M, N, K):
    """(config id, S) the library picks for a split-K decode of this shape."""
    cid, s = ctypes.c_int32(), ctypes.c_int32()
    _check(load().swiglu_packed_splitk_plan(handle, M, N, K, ctypes.byref(cid), ctypes.byref(s)),
           "swiglu_packed_splitk_plan")
    return cid.value, s.value


def swiglu_forward_packed_splitk(handle, A, P, Y, M, N, K, workspace, ksplit=0, config_id=-1,
                                 stream=None):
    """Decode forward (M <= 16) on fragment-ordered W_fused P with K split over
    workgroups; `workspace` (a byte tensor, zeroed before its first use) holds
    the counters and fp32 partials."""
    _check(load().swiglu_forward_packed_splitk(handle, _ptr(A), _ptr(P), _ptr(Y), M, N, K,
                                               config_id, ksplit, _ptr(workspace),
                                               0 if workspace is None else
                                               workspace.numel() * workspace.element_size(),
                                               _stream(stream)),
           "swiglu_forward_packed_splitk")


def swiglu_mx_packed_bytes(N: int, K: int) -> int:
    return int(load().swiglu_mx_packed_bytes(N, K))


def swiglu_pack_mx_fragments(handle, W8, P8, K, N, stream=None):
    _check(load().swiglu_pack_mx_fragments(handle, _ptr(W8), _ptr(P8), K, N, _stream(stream)),
           "swiglu_pack_mx_fragments")


def swiglu_quantize_mx(handle, X, Q, S, rows, K, ks, stream=None):
    _check(load().swiglu_quantize_mx(handle, _ptr(X), _ptr(Q), _ptr(S), rows, K, ks,
                                     _stream(stream)), "swiglu_quantize_mx")


def swiglu_pack_kmajor(handle, W1, W2, Wt, K, N, stream=None):
    _check(load().swiglu_pack_kmajor(handle, _ptr(W1), _ptr(W2), _ptr(Wt), K, N,
                                     _stream(stream)), "swiglu_pack_kmajor")


def mx_scale_stride(K: int) -> int:
    """Row stride (bytes) of MX scale tensors used by this package: K/32 rounded up to 16."""
    return -(-(K // 32) // 16) * 16


def swiglu_quantize_fp8(handle, X, Q, count, inv_scale=1.0, stream=None):
    _check(load().swiglu_quantize_fp8(handle, _ptr(X), _ptr(Q), count, inv_scale,
                                      _stream(stream)), "swiglu_quantize_fp8")


def swiglu_pack_fp8(handle, W1, W2, W8, K, N, stream=None):
    _check(load().swiglu_pack_fp8(handle, _ptr(W1), _ptr(W2), _ptr(W8), K, N, _stream(stream)),
           "swiglu_pack_fp8")


def swiglu_query_fp8(handle, M, N, K, variant=VARIANT_AUTO):
    t = Tile()
    _check(load().swiglu_query_fp8(handle, M, N, K, variant, ctypes.byref(t)),
           "swiglu_query_fp8")
    return t.as_dict()


def swiglu_config_count() -> int:
    return load().swiglu_config_count()


def swiglu_config_info(config_id: int) -> dict:
    t = Tile()
    _check(load().swiglu_config_info(config_id, ctypes.byref(t)), "swiglu_config_info")
    return t.as_dict()


class Handle:
    """Owns a library handle; the calls take torch tensors (bf16 or int16 views)."""

    def __init__(self, device: int = 0):
        self.h = swiglu_create(device)

    def close(self):
        if self.h:
            swiglu_destroy(self.h)
            self.h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):  # pragma: no cover
        try:
            self.close()
        except Exception:
            pass
