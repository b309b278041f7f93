"""CPU oracle for the fused SwiGLU MLP GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import, link or call it, and it imports nothing from them: the two sides
meet only in the tests, through the bf16 bit patterns the seeded input
generator produces.

The arithmetic lives in ``oracle.c`` (plain C, fp32, k-ascending sums, no FMA
contraction), which follows the gist.science page "Riepilogo Tecnico:
Sovrapposizione delle Attivazioni a Livello di Tile per l'Inferenza Efficiente
di LLM" (summary of arXiv 2607.02521):

* §Definizione del Problema -- Y = SiLU(A x W1) (.) (A x W2);
* §Metodologia, Kernel-2 -- W_fused [K, 2N], Gate in even, Up in odd columns;
* §Contributi Chiave, item 3 -- accuracy is judged against an FP32 reference;
* §Definizione del Problema names FP8 quantisation, and the page "Ottimizzazione
  delle GEMM: la chiave per l'efficienza dei Large Language Models" MXFP8: the
  FP8 functions below read that as OCP E4M3 codes with per-tensor scales.

This module only marshals numpy arrays to the C functions.  Every function
here is pinned by CPU tests against facts that do not come from it (exact
brute force, closed forms, invariants, a float64 cross-check).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

LAYOUT_SEPARATE = 0
LAYOUT_INTERLEAVED = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (fp32, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    p, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    for name in ("oracle_swiglu_rows", "oracle_swiglu_cols"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, p, c_int, i64, i64, i64, p, i64, p, p, p, c_int]
        fn.restype = c_int
    lib.oracle_silu.argtypes = [p, p, i64]
    lib.oracle_gate.argtypes = [p, p, p, i64]
    lib.oracle_round_bf16.argtypes = [p, p, i64]
    lib.oracle_decode_bf16.argtypes = [p, p, i64]
    lib.oracle_pack_interleaved.argtypes = [p, p, p, i64, i64]
    lib.oracle_decode_e4m3.argtypes = [p, p, i64]
    lib.oracle_quantize_e4m3.argtypes = [p, ctypes.c_float, p, i64]
    lib.oracle_pack_fp8_kmajor.argtypes = [p, p, p, i64, i64]
    for fn in (lib.oracle_silu, lib.oracle_gate, lib.oracle_round_bf16,
               lib.oracle_decode_bf16, lib.oracle_pack_interleaved, lib.oracle_decode_e4m3,
               lib.oracle_quantize_e4m3, lib.oracle_pack_fp8_kmajor):
        fn.restype = None
    lib.oracle_quantize_mx.argtypes = [p, i64, i64, i64, p, p]
    lib.oracle_decode_mx.argtypes = [p, p, i64, i64, i64, p]
    lib.oracle_pack_kmajor_bf16.argtypes = [p, p, p, i64, i64]
    lib.oracle_pack_fragments.argtypes = [p, p, p, i64, i64]
    lib.oracle_pack_fp8_fragments.argtypes = [p, p, i64, i64]
    lib.oracle_pack_mx_fragments.argtypes = [p, p, i64, i64]
    for fn in (lib.oracle_quantize_mx, lib.oracle_decode_mx, lib.oracle_pack_kmajor_bf16,
               lib.oracle_pack_fragments, lib.oracle_pack_fp8_fragments,
               lib.oracle_pack_mx_fragments):
        fn.restype = None
    lib.oracle_swiglu_mx_rows.argtypes = [p, p, p, p, i64, i64, i64, i64, p, i64, p, p, p,
                                          c_int]
    lib.oracle_swiglu_mx_rows.restype = c_int
    f32 = ctypes.c_float
    lib.oracle_swiglu_fp8_rows.argtypes = [p, p, p, i64, i64, i64, f32, f32, f32, p, i64,
                                           p, p, p, c_int]
    lib.oracle_swiglu_fp8_rows.restype = c_int
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _u16(x, name):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError(f"{name} must hold bf16 bit patterns as uint16, got {x.dtype}")
    return x


def _ptr(x):
    return None if x is None else x.ctypes.data


def _shapes(a, w1, w2, layout):
    a = _u16(a, "A")
    M, K = a.shape
    w1 = _u16(w1, "W1")
    if layout == LAYOUT_INTERLEAVED:
        if w1.shape[0] != K or w1.shape[1] % 2:
            raise ValueError("W_fused must be [K, 2N]")
        N = w1.shape[1] // 2
        w2 = None
    else:
        w2 = _u16(w2, "W2")
        if w1.shape != w2.shape or w1.shape[0] != K:
            raise ValueError("W1 and W2 must both be [K, N]")
        N = w1.shape[1]
    return a, w1, w2, M, N, K


def swiglu_rows(a, w1, w2=None, layout=LAYOUT_SEPARATE, rows=None,
                with_gate_up=False, nthreads=None):
    """fp32 y = SiLU(g) * u (and optionally g, u) for the listed rows.

    a: uint16 [M, K]; w1, w2: uint16 [K, N] (separate) or w1 = W_fused
    uint16 [K, 2N] (interleaved).  Returns y [len(rows), N] (all rows when
    rows is None), or (y, g, u).
    """
    a, w1, w2, M, N, K = _shapes(a, w1, w2, layout)
    lib = _load()
    if rows is None:
        ridx, nr = None, M
    else:
        ridx = np.ascontiguousarray(rows, dtype=np.int64)
        nr = ridx.size
    y = np.empty((nr, N), np.float32)
    g = np.empty((nr, N), np.float32) if with_gate_up else None
    u = np.empty((nr, N), np.float32) if with_gate_up else None
    rc = lib.oracle_swiglu_rows(_ptr(a), _ptr(w1), _ptr(w2), layout, M, N, K,
                                _ptr(ridx), nr, _ptr(y), _ptr(g), _ptr(u),
                                nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle_swiglu_rows rejected its arguments")
    return (y, g, u) if with_gate_up else y


def swiglu_cols(a, w1, w2=None, layout=LAYOUT_SEPARATE, cols=(),
                with_gate_up=False, nthreads=None):
    """fp32 y (and optionally g, u) for every row and the listed columns: [M, len(cols)]."""
    a, w1, w2, M, N, K = _shapes(a, w1, w2, layout)
    lib = _load()
    cidx = np.ascontiguousarray(cols, dtype=np.int64)
    nc = cidx.size
    y = np.empty((M, nc), np.float32)
    g = np.empty((M, nc), np.float32) if with_gate_up else None
    u = np.empty((M, nc), np.float32) if with_gate_up else None
    rc = lib.oracle_swiglu_cols(_ptr(a), _ptr(w1), _ptr(w2), layout, M, N, K,
                                _ptr(cidx), nc, _ptr(y), _ptr(g), _ptr(u),
                                nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle_swiglu_cols rejected its arguments")
    return (y, g, u) if with_gate_up else y


def swiglu(a, w1, w2=None, layout=LAYOUT_SEPARATE, nthreads=None):
    """fp32 y for the whole [M, N] output."""
    return swiglu_rows(a, w1, w2, layout, None, False, nthreads)


def silu(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    _load().oracle_silu(_ptr(x), _ptr(out), x.size)
    return out


def gate(g, u):
    """fp32 SiLU(g) * u element-wise."""
    g = np.ascontiguousarray(g, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.float32)
    if g.shape != u.shape:
        raise ValueError("g and u differ in shape")
    y = np.empty_like(g)
    _load().oracle_gate(_ptr(g), _ptr(u), _ptr(y), g.size)
    return y


def round_bf16(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_bf16(_ptr(x), _ptr(out), x.size)
    return out


def decode_bf16(x):
    """bf16 bit patterns (uint16) -> exact fp32."""
    x = _u16(x, "x")
    out = np.empty(x.shape, np.float32)
    _load().oracle_decode_bf16(_ptr(x), _ptr(out), x.size)
    return out


def pack_interleaved(w1, w2):
    """W_fused [K, 2N] from W1, W2 [K, N]: even columns Gate, odd columns Up."""
    w1 = _u16(w1, "W1")
    w2 = _u16(w2, "W2")
    if w1.shape != w2.shape:
        raise ValueError("W1 and W2 differ in shape")
    K, N = w1.shape
    wf = np.empty((K, 2 * N), np.uint16)
    _load().oracle_pack_interleaved(_ptr(w1), _ptr(w2), _ptr(wf), K, N)
    return wf


def swiglu_unfused_emulation(a, w1, w2, rows=None, nthreads=None):
    """What an unfused pipeline that stores Gate and Up as bf16 computes.

    Returns (y_fp32, g_bf16_bits, u_bf16_bits): y = SiLU(bf16(g)) * bf16(u) in
    fp32, for the listed rows (all when None).  The page's baseline writes both
    intermediates to HBM between the GEMMs and the activation (§Definizione
    del Problema); bf16 is the storage type of those tensors here.
    """
    _, g, u = swiglu_rows(a, w1, w2, LAYOUT_SEPARATE, rows, True, nthreads)
    gb, ub = round_bf16(g), round_bf16(u)
    return gate(decode_bf16(gb), decode_bf16(ub)), gb, ub


# ---- FP8 (OCP E4M3) inputs --------------------------------------------------
# Reading of the pages (they name FP8 and MXFP8 but fix no encoding): OCP E4M3
# codes with one fp32 scale per tensor, a code q standing for scale * decode(q).
# The arithmetic is in oracle.c.


def _u8(x, name):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint8:
        raise TypeError(f"{name} must hold E4M3 codes as uint8, got {x.dtype}")
    return x


def decode_e4m3(x):
    """E4M3 codes (uint8) -> exact float64 values (NaN for S.1111.111)."""
    x = _u8(x, "x")
    out = np.empty(x.shape, np.float64)
    _load().oracle_decode_e4m3(_ptr(x), _ptr(out), x.size)
    return out


def quantize_e4m3(x, inv_scale=1.0):
    """fp32 values -> E4M3 codes of fp32(x * inv_scale), nearest-even, saturating at 448."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().oracle_quantize_e4m3(_ptr(x), float(np.float32(inv_scale)), _ptr(out), x.size)
    return out


def pack_fp8_kmajor(w1, w2):
    """W8 [2N, K] from W1, W2 [K, N] E4M3: row 2n = Gate column n, row 2n+1 = Up column n."""
    w1 = _u8(w1, "W1")
    w2 = _u8(w2, "W2")
    if w1.shape != w2.shape:
        raise ValueError("W1 and W2 differ in shape")
    K, N = w1.shape
    w8 = np.empty((2 * N, K), np.uint8)
    _load().oracle_pack_fp8_kmajor(_ptr(w1), _ptr(w2), _ptr(w8), K, N)
    return w8


def swiglu_fp8_rows(a, w1, w2, s_a=1.0, s_w1=1.0, s_w2=1.0, rows=None,
                    with_gate_up=False, nthreads=None):
    """fp32 y = SiLU(g) * u of the FP8 forward (and optionally g, u) for the listed rows.

    a: uint8 E4M3 [M, K]; w1, w2: uint8 E4M3 [K, N]; s_*: the per-tensor fp32
    scales.  g = s_a s_w1 (exact dot product of the decoded codes), rounded to fp32.
    """
    a = _u8(a, "A")
    w1 = _u8(w1, "W1")
    w2 = _u8(w2, "W2")
    M, K = a.shape
    if w1.shape != w2.shape or w1.shape[0] != K:
        raise ValueError("W1 and W2 must both be [K, N]")
    N = w1.shape[1]
    lib = _load()
    if rows is None:
        ridx, nr = None, M
    else:
        ridx = np.ascontiguousarray(rows, dtype=np.int64)
        nr = ridx.size
    y = np.empty((nr, N), np.float32)
    g = np.empty((nr, N), np.float32) if with_gate_up else None
    u = np.empty((nr, N), np.float32) if with_gate_up else None
    f = lambda v: float(np.float32(v))
    rc = lib.oracle_swiglu_fp8_rows(_ptr(a), _ptr(w1), _ptr(w2), M, N, K, f(s_a), f(s_w1),
                                    f(s_w2), _ptr(ridx), nr, _ptr(y), _ptr(g), _ptr(u),
                                    nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle_swiglu_fp8_rows rejected its arguments")
    return (y, g, u) if with_gate_up else y


# ---- MXFP8 (OCP Microscaling, E4M3 elements, E8M0 scale per 32 along K) ------


def mx_scale_stride(K: int) -> int:
    """Row stride (bytes) of the E8M0 scale tensors: K/32 rounded up to 16."""
    return -(-(K // 32) // 16) * 16


def quantize_mx(x, ks=None):
    """fp32 rows [R, K] (K % 32 == 0) -> (E4M3 codes [R, K], E8M0 scales [R, ks])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    ks = mx_scale_stride(K) if ks is None else ks
    q = np.empty((R, K), np.uint8)
    s = np.empty((R, ks), np.uint8)
    _load().oracle_quantize_mx(_ptr(x), R, K, ks, _ptr(q), _ptr(s))
    return q, s


def decode_mx(q, s):
    """Real values (float64 [R, K]) of MX rows."""
    q = _u8(q, "q")
    s = _u8(s, "s")
    R, K = q.shape
    out = np.empty((R, K), np.float64)
    _load().oracle_decode_mx(_ptr(q), _ptr(s), R, K, s.shape[1], _ptr(out))
    return out


def pack_kmajor_bf16(w1, w2):
    """Wt [2N, K] (bf16 bits) from W1, W2 [K, N]: row 2n = W1[:, n], row 2n+1 = W2[:, n]."""
    w1 = _u16(w1, "W1")
    w2 = _u16(w2, "W2")
    if w1.shape != w2.shape:
        raise ValueError("W1 and W2 differ in shape")
    K, N = w1.shape
    wt = np.empty((2 * N, K), np.uint16)
    _load().oracle_pack_kmajor_bf16(_ptr(w1), _ptr(w2), _ptr(wt), K, N)
    return wt


def packed_size(N: int, K: int) -> int:
    """Values of the fragment-ordered W_fused: ceil(2N/128) * ceil(K/32) * 4096."""
    return ((2 * N + 127) // 128) * ((K + 31) // 32) * 4096


def pack_fragments(w1, w2):
    """Fragment-ordered W_fused (flat bf16 bits, packed_size(N, K) values) from
    W1, W2 [K, N]: element W_fused[k, j] at ((s*T + t)*8 + c)*512 + (16g + l)*8 + e
    (s = j // 128, l = j % 128 // 8, c = j % 8, t = k // 32, g = k % 32 // 8,
    e = k % 8, T = ceil(K/32)), zeros elsewhere."""
    w1 = _u16(w1, "W1")
    w2 = _u16(w2, "W2")
    if w1.shape != w2.shape:
        raise ValueError("W1 and W2 differ in shape")
    K, N = w1.shape
    out = np.empty(packed_size(N, K), np.uint16)
    _load().oracle_pack_fragments(_ptr(w1), _ptr(w2), _ptr(out), K, N)
    return out


def fp8_packed_size(N: int, K: int) -> int:
    """Bytes of the fragment-ordered W8: ceil(2N/16) * ceil(K/128) * 2048."""
    return ((2 * N + 15) // 16) * ((K + 127) // 128) * 2048


def pack_fp8_fragments(w8):
    """Fragment-ordered W8 (flat bytes, fp8_packed_size(N, K)) from W8 [2N, K]:
    byte W8[r, k] at ((rb*T + t)*2 + h)*1024 + (16g + i)*16 + e (rb = r // 16,
    i = r % 16, t = k // 128, h = k % 128 // 64, g = k % 64 // 16, e = k % 16,
    T = ceil(K/128)), zeros elsewhere."""
    w8 = _u8(w8, "W8")
    R, K = w8.shape
    out = np.empty(((R + 15) // 16) * ((K + 127) // 128) * 2048, np.uint8)
    _load().oracle_pack_fp8_fragments(_ptr(w8), _ptr(out), R, K)
    return out


def mx_packed_size(N: int, K: int) -> int:
    """Bytes of the MX fragment-ordered W8 (K % 64 == 0): ceil(2N/32) * (K/64) * 2048."""
    return ((2 * N + 31) // 32) * (K // 64) * 2048


def pack_mx_fragments(w8):
    """MX fragment-ordered W8 (flat bytes, mx_packed_size(N, K)) from W8 [2N, K]
    with K % 64 == 0: byte W8[r, k] at ((rb*T + t)*2 + v)*1024 + (i + 32h)*16 + e
    (rb = r // 32, i = r % 32, t = k // 64, v = k % 64 // 32, h = k % 32 // 16,
    e = k % 16, T = K/64), zeros elsewhere."""
    w8 = _u8(w8, "W8")
    R, K = w8.shape
    if K % 64:
        raise ValueError("K must be a multiple of 64")
    out = np.empty(((R + 31) // 32) * (K // 64) * 2048, np.uint8)
    _load().oracle_pack_mx_fragments(_ptr(w8), _ptr(out), R, K)
    return out


def swiglu_mx_rows(a, sa, w, sw, rows=None, with_gate_up=False, nthreads=None):
    """fp32 y of the MXFP8 forward (and optionally g, u) for the listed rows.

    a [M, K] E4M3 + sa [M, ks] E8M0; w [2N, K] E4M3 (row 2n Gate, 2n+1 Up) +
    sw [2N, ks].  The dot products are summed in fp64 over the decoded values.
    """
    a, sa, w, sw = _u8(a, "A"), _u8(sa, "SA"), _u8(w, "W"), _u8(sw, "SW")
    M, K = a.shape
    if w.shape[1] != K or w.shape[0] % 2 or sa.shape[0] != M or sw.shape[0] != w.shape[0] \
            or sa.shape[1] != sw.shape[1]:
        raise ValueError("shapes do not match")
    N = w.shape[0] // 2
    lib = _load()
    if rows is None:
        ridx, nr = None, M
    else:
        ridx = np.ascontiguousarray(rows, dtype=np.int64)
        nr = ridx.size
    y = np.empty((nr, N), np.float32)
    g = np.empty((nr, N), np.float32) if with_gate_up else None
    u = np.empty((nr, N), np.float32) if with_gate_up else None
    rc = lib.oracle_swiglu_mx_rows(_ptr(a), _ptr(sa), _ptr(w), _ptr(sw), M, N, K, sa.shape[1],
                                   _ptr(ridx), nr, _ptr(y), _ptr(g), _ptr(u),
                                   nthreads or default_threads())
    if rc < 0:
        raise ValueError("oracle_swiglu_mx_rows rejected its arguments")
    return (y, g, u) if with_gate_up else y
