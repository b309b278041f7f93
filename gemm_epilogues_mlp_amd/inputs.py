"""Seeded synthetic inputs for the SwiGLU MLP workloads.

This module holds no arithmetic of the method: it draws normal numbers with
numpy's PCG64, stores them as bf16 bit patterns (round to nearest even on the
fp32 bits) and lays them out.  Both the HIP path and the CPU oracle consume
exactly these bits; neither computes its inputs itself.

The shapes are the hidden/intermediate sizes of Qwen2.5 MLPs (0.5B, 1.5B,
7B decode, 7B prefill, 72B).  The page that defines the method evaluates on
Qwen-2.5 0.5B to 72B MLPs ("Riepilogo Tecnico: Sovrapposizione delle
Attivazioni a Livello di Tile...", §Risultati); no checkpoint is used, so
weights are random with the variance that keeps A.W ~ N(0, 1):
A ~ N(0, 1), W1, W2 ~ N(0, 1/K).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    index: int  # seeds are 1000 * index + tensor id

    @property
    def flops(self) -> int:
        """Two GEMMs of M x N x K, 2 flops per multiply-add."""
        return 4 * self.M * self.N * self.K

    @property
    def fused_bytes(self) -> int:
        """HBM bytes of the fused path: A, W1 + W2 and Y once each (bf16)."""
        return 2 * self.M * self.K + 4 * self.K * self.N + 2 * self.M * self.N

    @property
    def unfused_bytes(self) -> int:
        """A read by both GEMMs, weights once, Gate/Up written and read, Y."""
        return 4 * self.M * self.K + 4 * self.K * self.N + 10 * self.M * self.N


WORKLOADS = (
    Workload("qwen2.5-0.5b-mlp", 128, 896, 4864, 1),
    Workload("qwen2.5-1.5b-mlp", 2048, 1536, 8960, 2),
    Workload("qwen2.5-7b-mlp-decode", 16, 3584, 18944, 3),
    Workload("qwen2.5-7b-mlp-prefill", 8192, 3584, 18944, 4),
    Workload("qwen2.5-72b-mlp", 4096, 8192, 29568, 5),
)
BY_NAME = {w.name: w for w in WORKLOADS}

TENSOR_A, TENSOR_W1, TENSOR_W2 = 0, 1, 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    out = ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(seed: int, shape, scale: float, chunk_rows: int = 1024) -> np.ndarray:
    """Draw N(0, scale^2) in fp32 with PCG64(seed), round to bf16 bits.

    The draw is made in row chunks to bound host memory; the sequence equals
    a single draw of the whole array.
    """
    rng = np.random.default_rng(seed)
    rows, cols = shape
    out = np.empty(shape, np.uint16)
    s = np.float32(scale)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if scale != 1.0:
            x *= s
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def make_a(M: int, K: int, seed: int) -> np.ndarray:
    return _normal_bf16(seed, (M, K), 1.0)


def make_w(K: int, N: int, seed: int) -> np.ndarray:
    return _normal_bf16(seed, (K, N), float(1.0 / np.sqrt(np.float32(K))))


def make_inputs(M: int, K: int, N: int, index: int):
    """(A [M,K], W1 [K,N], W2 [K,N]) as uint16 bf16 bits, seeds 1000*index + t."""
    a = make_a(M, K, 1000 * index + TENSOR_A)
    w1 = make_w(K, N, 1000 * index + TENSOR_W1)
    w2 = make_w(K, N, 1000 * index + TENSOR_W2)
    return a, w1, w2


def workload_inputs(w: Workload):
    return make_inputs(w.M, w.K, w.N, w.index)


def interleave_columns(w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Column-interleave two [K, N] bit arrays into [K, 2N] (even <- w1, odd <- w2).

    A layout step only (no arithmetic): the storage format of the fused weight.
    """
    if w1.shape != w2.shape:
        raise ValueError("shape mismatch")
    K, N = w1.shape
    out = np.empty((K, 2 * N), w1.dtype)
    out[:, 0::2] = w1
    out[:, 1::2] = w2
    return out
