"""Pins of the oracle's fragment-ordered W_fused (CPU, no GPU).

The layout is the library's PACKED storage of the Kernel-2 matrix W_fused
("Riepilogo Tecnico: Sovrapposizione delle Attivazioni a Livello di Tile...",
§Metodologia, Kernel-2: Gate in even, Up in odd columns), cut into slabs of
128 columns and steps of 32 k:
    P[((s T + t) 8 + c) 512 + (16 g + l) 8 + e] = W_fused[32 t + 8 g + e][128 s + 8 l + c]
with zeros outside [K, 2N].  The oracle places every element by that rule.
Pinned here by positions derived by hand (tests/golden/fragment_layout.txt),
by the permutation property (every weight appears once, everything else is
zero), and by an independent derivation through numpy axis algebra on the
zero-padded W_fused.
"""
import os

import numpy as np
import pytest

import oracle
from gemm_epilogues_mlp_amd import inputs as I


def _golden():
    path = os.path.join(os.path.dirname(__file__), "golden", "fragment_layout.txt")
    entries, shape = [], None
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("shape"):
            shape = tuple(int(x) for x in line.split()[1:])
            continue
        i, v = line.split()
        entries.append((int(i), int(v)))
    return shape, entries


def _coded(K, N):
    k = np.arange(K, dtype=np.int64)[:, None]
    n = np.arange(N, dtype=np.int64)[None, :]
    return (1 + 72 * k + n).astype(np.uint16), (10001 + 72 * k + n).astype(np.uint16)


def test_hand_derived_positions():
    (K, N), entries = _golden()
    w1, w2 = _coded(K, N)
    p = oracle.pack_fragments(w1, w2)
    assert p.size == 16384 == oracle.packed_size(N, K)
    for i, v in entries:
        assert int(p[i]) == v, f"P[{i}] = {int(p[i])}, hand derivation says {v}"


@pytest.mark.parametrize("K,N", [(40, 72), (32, 64), (8, 8), (96, 264), (200, 72), (136, 120)])
def test_every_weight_once_zeros_elsewhere(K, N):
    rng = np.random.default_rng(K * 1000 + N)
    # distinct nonzero codes for all 2NK weights
    codes = rng.permutation(np.arange(1, 2 * N * K + 1, dtype=np.int64))
    assert codes.max() < 65536
    w1 = codes[:K * N].reshape(K, N).astype(np.uint16)
    w2 = codes[K * N:].reshape(K, N).astype(np.uint16)
    p = oracle.pack_fragments(w1, w2)
    assert p.size == ((2 * N + 127) // 128) * ((K + 31) // 32) * 4096
    nz = p[p != 0]
    assert nz.size == 2 * N * K
    assert np.array_equal(np.sort(nz.astype(np.int64)), np.sort(codes))


@pytest.mark.parametrize("K,N", [(40, 72), (64, 128), (8, 8), (200, 264), (520, 136),
                                 (3584, 64)])
def test_matches_axis_algebra(K, N):
    """Pad W_fused to [32T, 128S], split k as (t, g, e) and the column as
    (s, l, c), and order the axes (s, t, c, g, l, e)."""
    a, w1, w2 = I.make_inputs(1, K, N, 7)
    wf = I.interleave_columns(w1, w2)           # [K, 2N], Gate even, Up odd
    T, S = (K + 31) // 32, (2 * N + 127) // 128
    pad = np.zeros((32 * T, 128 * S), np.uint16)
    pad[:K, :2 * N] = wf
    ref = pad.reshape(T, 4, 8, S, 16, 8).transpose(3, 0, 5, 1, 4, 2).reshape(-1)
    assert np.array_equal(oracle.pack_fragments(w1, w2), ref)


def test_empty():
    w = np.zeros((0, 16), np.uint16)
    assert oracle.pack_fragments(w, w).size == 0


# ---- FP8: fragment-ordered W8 ------------------------------------------------
# W8 [2N, K] (E4M3 bytes, row 2n Gate, 2n+1 Up) cut into blocks of 16 rows and
# steps of 128 k, each 2 KB block stored as two 1 KB halves:
#   P8[((rb T + t) 2 + h) 1024 + (16 g + i) 16 + e] = W8[16 rb + i][128 t + 64 h + 16 g + e]


def _golden_fp8():
    path = os.path.join(os.path.dirname(__file__), "golden", "fp8_fragment_layout.txt")
    entries, shape = [], None
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("shape"):
            shape = tuple(int(x) for x in line.split()[1:])
            continue
        i, v = line.split()
        entries.append((int(i), int(v)))
    return shape, entries


def test_fp8_hand_derived_positions():
    (N, K), entries = _golden_fp8()
    r = np.arange(2 * N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    w8 = ((144 * r + k) % 251 + 1).astype(np.uint8)
    p = oracle.pack_fp8_fragments(w8)
    assert p.size == 8192 == oracle.fp8_packed_size(N, K)
    for i, v in entries:
        assert int(p[i]) == v, f"P8[{i}] = {int(p[i])}, hand derivation says {v}"


@pytest.mark.parametrize("N,K", [(12, 144), (8, 16), (64, 256), (36, 400), (100, 128)])
def test_fp8_every_byte_once_zeros_elsewhere(N, K):
    """Distinct 16-bit tags split over two byte planes: each (row, k) appears
    exactly once, padding is zero."""
    R = 2 * N
    tag = np.arange(1, R * K + 1, dtype=np.int64).reshape(R, K)
    assert tag.max() < 65536
    lo, hi = (tag & 0xFF).astype(np.uint8), (tag >> 8).astype(np.uint8)
    plo, phi = oracle.pack_fp8_fragments(lo), oracle.pack_fp8_fragments(hi)
    got = plo.astype(np.int64) | (phi.astype(np.int64) << 8)
    assert got.size == ((R + 15) // 16) * ((K + 127) // 128) * 2048
    nz = got[got != 0]
    assert nz.size == R * K
    assert np.array_equal(np.sort(nz), tag.reshape(-1))


@pytest.mark.parametrize("N,K", [(12, 144), (8, 16), (64, 256), (36, 400), (9472, 3584)])
def test_fp8_matches_axis_algebra(N, K):
    """Pad W8 to [16 RB, 128 T], split the row as (rb, i) and k as (t, h, g, e),
    and order the axes (rb, t, h, g, i, e)."""
    rng = np.random.default_rng(N + K)
    w8 = rng.integers(0, 256, (2 * N, K), dtype=np.uint8)
    RB, T = (2 * N + 15) // 16, (K + 127) // 128
    pad = np.zeros((16 * RB, 128 * T), np.uint8)
    pad[:2 * N, :K] = w8
    ref = pad.reshape(RB, 16, T, 2, 4, 16).transpose(0, 2, 3, 4, 1, 5).reshape(-1)
    assert np.array_equal(oracle.pack_fp8_fragments(w8), ref)


# ---- MXFP8: W8 in the 32x32x64 fragment order ------------------------------------
#   P8[((rb T + t) 2 + v) 1024 + (i + 32 h) 16 + e] = W8[32 rb + i][64 t + 32 v + 16 h + e]


def test_mx_hand_derived_positions():
    path = os.path.join(os.path.dirname(__file__), "golden", "mx_fragment_layout.txt")
    entries, shape = [], None
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        if line.startswith("shape"):
            shape = tuple(int(x) for x in line.split()[1:])
            continue
        i, v = line.split()
        entries.append((int(i), int(v)))
    N, K = shape
    r = np.arange(2 * N, dtype=np.int64)[:, None]
    k = np.arange(K, dtype=np.int64)[None, :]
    w8 = ((128 * r + k) % 251 + 1).astype(np.uint8)
    p = oracle.pack_mx_fragments(w8)
    assert p.size == 8192 == oracle.mx_packed_size(N, K)
    for i, v in entries:
        assert int(p[i]) == v, f"P8[{i}] = {int(p[i])}, hand derivation says {v}"


@pytest.mark.parametrize("N,K", [(20, 128), (8, 64), (64, 256), (36, 448), (100, 64)])
def test_mx_every_byte_once_zeros_elsewhere(N, K):
    R = 2 * N
    tag = np.arange(1, R * K + 1, dtype=np.int64).reshape(R, K)
    assert tag.max() < 65536
    lo, hi = (tag & 0xFF).astype(np.uint8), (tag >> 8).astype(np.uint8)
    got = oracle.pack_mx_fragments(lo).astype(np.int64) | \
        (oracle.pack_mx_fragments(hi).astype(np.int64) << 8)
    assert got.size == ((R + 31) // 32) * (K // 64) * 2048
    nz = got[got != 0]
    assert nz.size == R * K
    assert np.array_equal(np.sort(nz), tag.reshape(-1))


@pytest.mark.parametrize("N,K", [(20, 128), (8, 64), (64, 256), (36, 448), (9472, 3584)])
def test_mx_matches_axis_algebra(N, K):
    """Pad W8 to [32 RB, K], split the row as (rb, i) and k as (t, v, h, e),
    and order the axes (rb, t, v, h, i, e)."""
    rng = np.random.default_rng(N * 7 + K)
    w8 = rng.integers(0, 256, (2 * N, K), dtype=np.uint8)
    RB, T = (2 * N + 31) // 32, K // 64
    pad = np.zeros((32 * RB, K), np.uint8)
    pad[:2 * N] = w8
    ref = pad.reshape(RB, 32, T, 2, 2, 16).transpose(0, 2, 3, 4, 1, 5).reshape(-1)
    assert np.array_equal(oracle.pack_mx_fragments(w8), ref)
