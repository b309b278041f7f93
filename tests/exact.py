"""Exact brute-force references used to pin the oracle on tiny shapes.

A bf16 value has an 8-bit significand, so the product of two bf16 values has
at most 16 significant bits and is exact in float64; math.fsum then returns
the correctly rounded sum.  g and u below are therefore exact to half an ulp
of float64 -- far tighter than any fp32 computation -- and depend on nothing
in the oracle or the HIP library.
"""
import math

import numpy as np


def bf16_values(bits):
    """bf16 bit patterns -> float64 values (exact), via the fp32 bit layout."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def exact_dot_matrix(a_bits, w_bits):
    """[M, N] float64 of sum_k a[m,k] * w[k,n], each a correctly rounded fsum."""
    a = bf16_values(a_bits)
    w = bf16_values(w_bits)
    M, K = a.shape
    K2, N = w.shape
    assert K == K2
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            out[m, n] = math.fsum(a[m, k] * w[k, n] for k in range(K))
    return out


def abs_dot_matrix(a_bits, w_bits):
    """[M, N] of sum_k |a[m,k] * w[k,n]| (the scale in the summation error bound)."""
    a = np.abs(bf16_values(a_bits))
    w = np.abs(bf16_values(w_bits))
    return a @ w


def gamma(n, unit=2.0 ** -24):
    """Higham's gamma_n = n u / (1 - n u) for recursive summation in fp32."""
    return n * unit / (1.0 - n * unit)


def silu64(x):
    """SiLU(x) = x / (1 + e^-x) in float64, elementwise, overflow-safe."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))
