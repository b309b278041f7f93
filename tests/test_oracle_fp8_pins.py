"""Pins for the FP8 (OCP E4M3) part of the CPU oracle, from facts that do not
come from the oracle itself:

* the E4M3 decode against the format's anchor values (smallest subnormal,
  largest subnormal, smallest normal, one, largest finite, the NaN codes),
  its structural invariants, and PyTorch's own float8_e4m3fn decode;
* quantisation against an exhaustive nearest-value search (ties to the even
  code) over every bf16 bit pattern, and against PyTorch's float8_e4m3fn
  conversion wherever that conversion does not overflow;
* the FP8 forward against exact rational brute force on tiny shapes, against
  the bf16 oracle on the same values (every E4M3 value is a bf16 value), the
  A = I special case and the W2 = 0 and power-of-two scaling invariants.

The pages name FP8 and MXFP8 inputs ("Riepilogo Tecnico: Sovrapposizione delle
Attivazioni a Livello di Tile per l'Inferenza Efficiente di LLM",
§Definizione del Problema; "Ottimizzazione delle GEMM: la chiave per
l'efficienza dei Large Language Models", §Impatto sui deployment on-premise)
without fixing an encoding; the reading is OCP E4M3 with per-tensor scales.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from gemm_epilogues_mlp_amd import inputs as I

CODES = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


# --------------------------------------------------------------------------- decode
def test_decode_anchor_values():
    v = oracle.decode_e4m3(CODES)
    assert v[0x00] == 0.0 and not math.copysign(1.0, v[0x00]) < 0
    assert v[0x80] == 0.0 and math.copysign(1.0, v[0x80]) < 0
    assert v[0x01] == 2.0 ** -9           # smallest subnormal
    assert v[0x07] == 0.875 * 2.0 ** -6   # largest subnormal
    assert v[0x08] == 2.0 ** -6           # smallest normal
    assert v[0x38] == 1.0
    assert v[0x3F] == 1.875
    assert v[0x40] == 2.0
    assert v[0x7E] == 448.0               # largest finite
    assert v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2       # no infinities, two NaN codes


def test_decode_structure():
    v = oracle.decode_e4m3(CODES)
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes order the values
    assert np.array_equal(v[0x80:0xFF], -pos)            # sign-magnitude
    # within each binade the eight codes are evenly spaced by 2^(e-10)
    for e in range(1, 16):
        b = pos[8 * e: 8 * e + 8] if e < 15 else pos[8 * e: 8 * e + 7]
        assert np.all(np.diff(b) == 2.0 ** (e - 10))


def test_decode_matches_torch():
    v = oracle.decode_e4m3(CODES)
    t = torch_decode(CODES)
    fin = ~np.isnan(t)
    assert np.array_equal(np.isnan(v), ~fin)
    assert np.array_equal(v[fin], t[fin])
    assert np.array_equal(np.signbit(v[fin]), np.signbit(t[fin]))


# --------------------------------------------------------------------------- quantise
def nearest_code(x):
    """Exhaustive nearest-value search over the finite E4M3 codes (ties to the
    code with an even mantissa), saturating; NaN -> NaN code.  x: float64."""
    vals = torch_decode(CODES[:0x7F])                    # 0 .. 448, torch's decode
    out = np.empty(x.shape, np.uint8)
    for i, xi in enumerate(x):
        s = 0x80 if math.copysign(1.0, xi) < 0 else 0
        if math.isnan(xi):
            out[i] = s | 0x7F
            continue
        a = abs(xi)
        if a >= 448.0:            # nearest finite value of anything above the range
            out[i] = s | 0x7E
            continue
        d = np.abs(vals - a)      # exact near the minimum (Sterbenz)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        out[i] = s | c
    return out


@pytest.mark.parametrize("inv_scale", [1.0, 64.0, 0.001953125, 3.0])
def test_quantize_every_bf16_pattern(inv_scale):
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << 16).view(np.float32)
    q = oracle.quantize_e4m3(x, inv_scale)
    with np.errstate(invalid="ignore", over="ignore"):
        v = (x * np.float32(inv_scale)).astype(np.float64)  # the fp32 product, as specified
    assert np.array_equal(q, nearest_code(v))


def test_quantize_matches_torch_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 200.0)])
    x = x.astype(np.float32)
    x = x[np.abs(x) < 448.0]          # torch's conversion overflows to NaN above the range
    q = oracle.quantize_e4m3(x)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, t)


def test_quantize_saturates_and_keeps_sign():
    x = np.array([448.0, 463.9, 464.0, 1e30, np.inf, -np.inf, -1e-30, -0.0, np.nan], np.float32)
    q = oracle.quantize_e4m3(x)
    assert list(q[:6]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert q[6] == 0x80 and q[7] == 0x80
    assert q[8] == 0x7F


# --------------------------------------------------------------------------- pack
def test_pack_fp8_kmajor_is_transpose_interleave():
    rng = np.random.default_rng(1)
    w1 = rng.integers(0, 256, (37, 24), dtype=np.uint8)
    w2 = rng.integers(0, 256, (37, 24), dtype=np.uint8)
    w8 = oracle.pack_fp8_kmajor(w1, w2)
    assert w8.shape == (48, 37)
    assert np.array_equal(w8[0::2], w1.T) and np.array_equal(w8[1::2], w2.T)


# --------------------------------------------------------------------------- forward
def finite_codes(rng, shape, spread=1.0):
    """Random finite E4M3 codes of values ~ N(0, spread^2), via the oracle's quantiser."""
    return oracle.quantize_e4m3(rng.standard_normal(shape).astype(np.float32) * np.float32(spread))


def exact_forward(a, w1, w2, sa, s1, s2):
    """Exact g and u (Fractions) and y in float64 from exact g, u."""
    A = [[Fraction(float(v)) for v in row] for row in torch_decode(a)]
    W1 = [[Fraction(float(v)) for v in row] for row in torch_decode(w1)]
    W2 = [[Fraction(float(v)) for v in row] for row in torch_decode(w2)]
    M, K = a.shape
    N = w1.shape[1]
    G, U = np.empty((M, N)), np.empty((M, N))
    for m in range(M):
        for n in range(N):
            G[m, n] = float(Fraction(sa) * Fraction(s1) * sum(A[m][k] * W1[k][n] for k in range(K)))
            U[m, n] = float(Fraction(sa) * Fraction(s2) * sum(A[m][k] * W2[k][n] for k in range(K)))
    with np.errstate(over="ignore"):
        Y = G / (1.0 + np.exp(-G)) * U
    return G, U, Y


@settings(max_examples=40, deadline=None)
@given(M=st.integers(1, 5), N=st.integers(1, 6), K=st.integers(1, 40),
       seed=st.integers(0, 2 ** 31 - 1),
       scales=st.sampled_from([(1.0, 1.0, 1.0), (0.5, 0.03125, 2.0), (0.1, 0.37, 1.7)]))
def test_fp8_forward_matches_exact_brute_force(M, N, K, seed, scales):
    rng = np.random.default_rng(seed)
    a = finite_codes(rng, (M, K), 4.0)
    w1 = finite_codes(rng, (K, N), 100.0)   # spans subnormals to 448
    w2 = finite_codes(rng, (K, N), 0.01)
    sa, s1, s2 = (float(np.float32(s)) for s in scales)
    y, g, u = oracle.swiglu_fp8_rows(a, w1, w2, sa, s1, s2, with_gate_up=True, nthreads=2)
    G, U, Y = exact_forward(a, w1, w2, sa, s1, s2)
    # g, u: the exact value rounded to fp32 (two roundings: fp64, then fp32)
    ulp = lambda x: np.spacing(np.abs(x).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(g - G) <= ulp(G) + 1e-44)
    assert np.all(np.abs(u - U) <= ulp(U) + 1e-44)
    # y: fp32 SiLU and product of those, a few fp32 roundings of |y| plus the
    # propagated rounding of g (|SiLU'| <= 1.1) and u
    bound = 1.1 * ulp(G) * np.abs(U) + np.abs(G) * ulp(U) + 2.0 ** -20 * np.abs(Y) + 1e-40
    assert np.all(np.abs(y - Y) <= bound)


def test_fp8_forward_equals_bf16_oracle_on_the_same_values():
    """Unit scales: the FP8 forward is the bf16 forward of the decoded values
    (each is exactly a bf16 value); only the fp32 summation order differs."""
    rng = np.random.default_rng(11)
    M, K, N = 6, 512, 40
    a = finite_codes(rng, (M, K))
    w1 = finite_codes(rng, (K, N), 1.0 / math.sqrt(K))
    w2 = finite_codes(rng, (K, N), 1.0 / math.sqrt(K))
    as_bf16 = lambda c: oracle.round_bf16(oracle.decode_e4m3(c).astype(np.float32))
    assert np.array_equal(oracle.decode_bf16(as_bf16(w1)), oracle.decode_e4m3(w1))
    y8, g8, u8 = oracle.swiglu_fp8_rows(a, w1, w2, with_gate_up=True, nthreads=2)
    yb, gb, ub = oracle.swiglu_rows(as_bf16(a), as_bf16(w1), as_bf16(w2), with_gate_up=True,
                                    nthreads=2)
    S = np.abs(oracle.decode_e4m3(a)) @ np.abs(oracle.decode_e4m3(w1))
    gam = K * 2.0 ** -24 / (1 - K * 2.0 ** -24)
    assert np.all(np.abs(g8 - gb) <= gam * S + np.spacing(np.abs(g8)))
    assert np.allclose(y8, yb, rtol=1e-4, atol=1e-5)


def test_fp8_identity_rows_copy_the_weights():
    """A = I (code 0x38 = 1.0 on the diagonal): g = s_a s_w1 w1 exactly."""
    rng = np.random.default_rng(3)
    K, N = 24, 16
    a = np.zeros((K, K), np.uint8)
    a[np.arange(K), np.arange(K)] = 0x38
    w1 = finite_codes(rng, (K, N), 8.0)
    w2 = finite_codes(rng, (K, N), 8.0)
    y, g, u = oracle.swiglu_fp8_rows(a, w1, w2, 0.5, 0.25, 2.0, with_gate_up=True)
    assert np.array_equal(g, (oracle.decode_e4m3(w1) * 0.125).astype(np.float32))
    assert np.array_equal(u, oracle.decode_e4m3(w2).astype(np.float32))


def test_fp8_invariants():
    rng = np.random.default_rng(4)
    M, K, N = 7, 96, 24
    a = finite_codes(rng, (M, K))
    w1 = finite_codes(rng, (K, N), 0.1)
    w2 = finite_codes(rng, (K, N), 0.1)
    y = oracle.swiglu_fp8_rows(a, w1, w2, 1.0, 1.0, 1.0)
    assert np.all(oracle.swiglu_fp8_rows(a, w1, np.zeros_like(w2)) == 0)
    assert np.all(oracle.swiglu_fp8_rows(a, np.zeros_like(w1), w2) == 0)
    # a power-of-two scale of W2 scales Y by it, bit for bit
    assert np.array_equal(oracle.swiglu_fp8_rows(a, w1, w2, 1.0, 1.0, 8.0), y * 8)
    # rows can be listed in any order
    rows = np.array([5, 0, 3])
    assert np.array_equal(oracle.swiglu_fp8_rows(a, w1, w2, rows=rows), y[rows])


# --------------------------------------------------------------------------- MXFP8
# OCP Microscaling reading: E4M3 elements, one E8M0 scale (2^(e-127)) per 32
# consecutive k; shared exponent floor(log2 max|V|) - 8, clamped to [-127, 127].
def test_decode_mx_anchor_values():
    q = np.array([[0x38] * 32 + [0x40] * 32], np.uint8)
    for e, f in [(127, 1.0), (128, 2.0), (0, 2.0 ** -127), (254, 2.0 ** 127)]:
        s = np.array([[e, 127] + [0] * 14], np.uint8)
        v = oracle.decode_mx(q, s)
        assert np.all(v[0, :32] == f) and np.all(v[0, 32:] == 2.0)
    v = oracle.decode_mx(q, np.array([[255, 127] + [0] * 14], np.uint8))
    assert np.all(np.isnan(v[0, :32])) and np.all(v[0, 32:] == 2.0)


def test_quantize_mx_hand_cases():
    x = np.zeros((4, 64), np.float32)
    x[0, :32] = 448.0                     # max 448: shared exponent 0 (e = 127), codes unchanged
    x[0, 32:] = 1.0                       # max 1: shared -8 (e = 119), 1 -> 256 = code 0x78
    x[1, 3] = -3.0                        # one non-zero: shared floor(log2 3) - 8 = -7
    x[2, :] = 2.0 ** -140                 # tiny: shared clamped to -127 (e = 0)
    q, s = oracle.quantize_mx(x)
    assert s.shape == (4, 16)
    assert list(s[0, :2]) == [127, 119] and np.all(q[0, :32] == 0x7E) and np.all(q[0, 32:] == 0x78)
    assert s[1, 0] == 120 and q[1, 3] == (0x80 | oracle.quantize_e4m3(np.float32([3 * 128.0]))[0])
    assert s[1, 1] == 0 and np.all(q[1, 32:] == 0)          # all-zero block: e = 0, codes 0
    assert s[2, 0] == 0
    assert np.all(s[:, 2:] == 0)                             # padding bytes of the scale rows
    y = np.zeros((1, 64), np.float32)
    y[0, 0], y[0, 1] = np.inf, 1.0                           # infinity counts as 2^128
    y[0, 32], y[0, 33] = np.nan, 2.0                         # NaN is left out of the maximum
    q, s = oracle.quantize_mx(y)
    assert s[0, 0] == 127 + 120 and q[0, 0] == 0x7E and q[0, 1] == 0
    assert s[0, 1] == 127 - 7 and q[0, 32] == 0x7F and q[0, 33] == 0x78


@settings(max_examples=30, deadline=None)
@given(seed=st.integers(0, 2 ** 31 - 1), spread=st.sampled_from([1e-3, 1.0, 37.0, 1e5]))
def test_quantize_mx_against_exhaustive_search(seed, spread):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, 96)) * spread).astype(np.float32)
    q, s = oracle.quantize_mx(x)
    for r in range(3):
        for b in range(3):
            v = x[r, 32 * b: 32 * b + 32].astype(np.float64)
            X = 2.0 ** (int(s[r, b]) - 127)
            # the largest magnitude lands in E4M3's top binade [256, 512)
            assert 256.0 <= np.max(np.abs(v)) / X < 512.0
            assert np.array_equal(q[r, 32 * b: 32 * b + 32], nearest_code(v / X))


def test_pack_kmajor_bf16_is_transpose_interleave():
    rng = np.random.default_rng(2)
    w1 = rng.integers(0, 65536, (40, 24), dtype=np.uint16)
    w2 = rng.integers(0, 65536, (40, 24), dtype=np.uint16)
    wt = oracle.pack_kmajor_bf16(w1, w2)
    assert wt.shape == (48, 40)
    assert np.array_equal(wt[0::2], w1.T) and np.array_equal(wt[1::2], w2.T)


def mx_case(rng, M, N, K):
    a = rng.standard_normal((M, K)).astype(np.float32) * np.float32(3.0)
    w = (rng.standard_normal((2 * N, K)) / np.sqrt(K)).astype(np.float32)
    w[:, :32] *= np.float32(50.0)                      # blocks of very different scale
    (qa, sa), (qw, sw) = oracle.quantize_mx(a), oracle.quantize_mx(w)
    return qa, sa, qw, sw


def test_mx_forward_with_unit_scales_equals_fp8_forward():
    rng = np.random.default_rng(12)
    M, N, K = 5, 24, 128
    qa, sa, qw, sw = mx_case(rng, M, N, K)
    y_mx, g_mx, u_mx = oracle.swiglu_mx_rows(qa, np.full_like(sa, 127), qw,
                                             np.full_like(sw, 127), with_gate_up=True)
    y8, g8, u8 = oracle.swiglu_fp8_rows(qa, np.ascontiguousarray(qw[0::2].T),
                                        np.ascontiguousarray(qw[1::2].T), with_gate_up=True)
    assert np.array_equal(g_mx, g8) and np.array_equal(u_mx, u8) and np.array_equal(y_mx, y8)


@settings(max_examples=25, deadline=None)
@given(M=st.integers(1, 4), N=st.integers(1, 5), KB=st.integers(1, 3),
       seed=st.integers(0, 2 ** 31 - 1))
def test_mx_forward_matches_exact_brute_force(M, N, KB, seed):
    K = 32 * KB
    rng = np.random.default_rng(seed)
    qa, sa, qw, sw = mx_case(rng, M, N, K)
    y, g, u = oracle.swiglu_mx_rows(qa, sa, qw, sw, with_gate_up=True, nthreads=2)
    A = [[Fraction(float(v)) for v in row] for row in torch_decode(qa)]
    Wv = [[Fraction(float(v)) for v in row] for row in torch_decode(qw)]
    SA = lambda m, k: Fraction(2) ** (int(sa[m, k // 32]) - 127)
    SW = lambda r, k: Fraction(2) ** (int(sw[r, k // 32]) - 127)
    ulp = lambda x: np.spacing(np.abs(np.float32(x))).astype(np.float64)
    for m in range(M):
        for n in range(N):
            G = float(sum(SA(m, k) * A[m][k] * SW(2 * n, k) * Wv[2 * n][k] for k in range(K)))
            U = float(sum(SA(m, k) * A[m][k] * SW(2 * n + 1, k) * Wv[2 * n + 1][k]
                          for k in range(K)))
            assert abs(g[m, n] - G) <= ulp(G) and abs(u[m, n] - U) <= ulp(U)
            with np.errstate(over="ignore"):
                Y = G / (1.0 + np.exp(-G)) * U
            assert abs(y[m, n] - Y) <= 1.1 * ulp(G) * abs(U) + abs(G) * ulp(U) + 2.0 ** -20 * abs(Y) + 1e-40


def test_mx_up_scale_doubles_y():
    rng = np.random.default_rng(13)
    qa, sa, qw, sw = mx_case(rng, 4, 16, 96)
    y = oracle.swiglu_mx_rows(qa, sa, qw, sw)
    sw2 = sw.copy()
    sw2[1::2, :3] += 1                                   # every Up block scale x 2
    assert np.array_equal(oracle.swiglu_mx_rows(qa, sa, qw, sw2), y * 2)
    sw0 = sw.copy()
    qw0 = qw.copy()
    qw0[1::2] = 0                                        # Up = 0 -> Y = 0
    assert np.all(oracle.swiglu_mx_rows(qa, sa, qw0, sw0) == 0)
