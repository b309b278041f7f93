"""Pins for the CPU oracle: facts that do not come from the oracle itself.

* exact brute force (correctly rounded float64 sums of exact products) on tiny
  shapes, within the fp32 recursive-summation error bound;
* SiLU closed forms;
* the A = I special case (no accumulation at all);
* invariants: W1 = 0 or W2 = 0 gives 0, interleaved equals separate bit for
  bit, row/column permutation equivariance, scaling W2 by 2^k scales Y by 2^k,
  row mode equals column mode bit for bit;
* round-to-nearest-even checked against the definition of the rounding;
* a float64 cross-check of full-size rows.

The method: "Riepilogo Tecnico: Sovrapposizione delle Attivazioni a Livello di
Tile per l'Inferenza Efficiente di LLM" -- §Definizione del Problema (the
formula), §Metodologia/Kernel-2 (W_fused pairing), §Contributi Chiave item 3
(FP32 reference).
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle
from exact import abs_dot_matrix, bf16_values, exact_dot_matrix, gamma, silu64
from gemm_epilogues_mlp_amd import inputs as I


def rand_bits(rng, shape, scale=1.0):
    return I.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def y_bound(g, u, Sg, Su, K):
    """Worst-case |y_oracle - y_exact| for fp32 summation + fp32 SiLU and product.

    |dg| <= gamma_K * sum|a w1|, |du| <= gamma_K * sum|a w2|; |SiLU'| <= 1.1;
    SiLU evaluation and the final product add a few fp32 roundings of |y|.
    """
    s = silu64(g)
    Eg = gamma(K) * Sg
    Eu = gamma(K) * Su
    return 1.1 * Eg * (np.abs(u) + Eu) + np.abs(s) * Eu + 2.0 ** -20 * np.abs(s * u) + 1e-37


# --------------------------------------------------------------------------- brute force
@settings(max_examples=60, deadline=None)
@given(M=st.integers(1, 9), N=st.integers(1, 9), K=st.integers(1, 40),
       seed=st.integers(0, 2 ** 31 - 1), scale=st.sampled_from([1.0, 0.05, 3.0]))
def test_oracle_matches_exact_brute_force(M, N, K, seed, scale):
    rng = np.random.default_rng(seed)
    a = rand_bits(rng, (M, K))
    w1 = rand_bits(rng, (K, N), scale / math.sqrt(K))
    w2 = rand_bits(rng, (K, N), scale / math.sqrt(K))
    y, g, u = oracle.swiglu_rows(a, w1, w2, with_gate_up=True, nthreads=2)
    ge = exact_dot_matrix(a, w1)
    ue = exact_dot_matrix(a, w2)
    Sg = abs_dot_matrix(a, w1)
    Su = abs_dot_matrix(a, w2)
    assert np.all(np.abs(g - ge) <= gamma(K) * Sg + 1e-37)
    assert np.all(np.abs(u - ue) <= gamma(K) * Su + 1e-37)
    ye = silu64(ge) * ue
    assert np.all(np.abs(y - ye) <= y_bound(ge, ue, Sg, Su, K))


def test_oracle_hand_cases():
    # K = 1: g = a*w1, u = a*w2 exactly; y = SiLU(a w1) * a w2.
    a = I.f32_to_bf16_bits(np.array([[2.0], [-1.5]], np.float32))
    w1 = I.f32_to_bf16_bits(np.array([[0.5, -1.0, 0.0]], np.float32))
    w2 = I.f32_to_bf16_bits(np.array([[3.0, 0.25, 7.0]], np.float32))
    y = oracle.swiglu(a, w1, w2).astype(np.float64)
    g = np.array([[1.0, -2.0, 0.0], [-0.75, 1.5, -0.0]])
    u = np.array([[6.0, 0.5, 14.0], [-4.5, -0.375, -10.5]])
    expect = silu64(g) * u
    assert np.allclose(y, expect, rtol=4 * 2.0 ** -23, atol=0)
    # M = N = 1 with cancellation: 1*1 + 1*(-1) + 2^-8 * 1 = 2^-8 exactly.
    a = I.f32_to_bf16_bits(np.array([[1.0, 1.0, 2.0 ** -8]], np.float32))
    w = I.f32_to_bf16_bits(np.array([[1.0], [-1.0], [1.0]], np.float32))
    _, g, u = oracle.swiglu_rows(a, w, w, with_gate_up=True)
    assert g[0, 0] == 2.0 ** -8 and u[0, 0] == 2.0 ** -8


def test_worked_example_fixture():
    """tests/golden/worked_example.txt: small dyadic inputs whose g, u are exact."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")
    blocks = {}
    cur = None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        if line.endswith(":"):
            cur = line[:-1]
            blocks[cur] = []
        else:
            blocks[cur].append([float(v) for v in line.split()])
    A = np.array(blocks["A"], np.float32)
    W1 = np.array(blocks["W1"], np.float32)
    W2 = np.array(blocks["W2"], np.float32)
    WF = np.array(blocks["W_fused"], np.float32)
    a, w1, w2 = (I.f32_to_bf16_bits(x) for x in (A, W1, W2))
    # the fixture's W_fused is the page's interleave written out by hand
    assert np.array_equal(oracle.pack_interleaved(w1, w2), I.f32_to_bf16_bits(WF))
    g = A.astype(np.float64) @ W1.astype(np.float64)   # exact: small dyadic values
    u = A.astype(np.float64) @ W2.astype(np.float64)
    y = oracle.swiglu(a, w1, w2).astype(np.float64)
    assert np.allclose(y, silu64(g) * u, rtol=4 * 2.0 ** -23, atol=1e-30)
    yi = oracle.swiglu(a, I.f32_to_bf16_bits(WF), layout=oracle.LAYOUT_INTERLEAVED)
    assert np.array_equal(yi.view(np.uint32), y.astype(np.float32).view(np.uint32))


# --------------------------------------------------------------------------- SiLU closed forms
def test_silu_closed_forms():
    ln3 = math.log(3.0)
    # sigma(ln 3) = 3/4, so SiLU(ln 3) = 0.75 ln 3
    xs = np.array([0.0, 1.0, ln3, -1.278464542761074, 2.0, -1.0, 30.0, -30.0], np.float32)
    out = oracle.silu(xs).astype(np.float64)
    x64 = xs.astype(np.float64)
    expect = np.array([
        0.0,
        1.0 / (1.0 + math.exp(-1.0)),           # 0.7310585786300049
        float(np.float32(ln3)) * (1.0 / (1.0 + math.exp(-float(np.float32(ln3))))),
        float("nan"),                            # minimum, checked below
        2.0 / (1.0 + math.exp(-2.0)),
        -1.0 / (1.0 + math.exp(1.0)),
        30.0 / (1.0 + math.exp(-30.0)),
        -30.0 / (1.0 + math.exp(30.0)),
    ])
    assert out[0] == 0.0
    assert abs(out[1] - 0.7310585786300049) <= 2 * 2.0 ** -24
    assert abs(out[2] - 0.75 * ln3) <= 3 * 2.0 ** -24  # includes rounding of ln 3 to fp32
    for i in (1, 2, 4, 5, 6, 7):
        assert abs(out[i] - expect[i]) <= 3 * 2.0 ** -24 * abs(expect[i]) + 1e-45
    # minimum of SiLU: x* = -1 - W0(1/e), SiLU(x*) = x* + 1 = -W0(1/e)
    assert abs(out[3] - (-0.2784645427610738)) <= 2.0 ** -22
    grid = np.linspace(-1.5, -1.05, 2001, dtype=np.float32)
    sg = oracle.silu(grid)
    assert abs(float(grid[np.argmin(sg)]) - (-1.278464542761074)) < 1e-3
    assert float(sg.min()) >= -0.2784645427610738 - 2.0 ** -22
    # odd/even split: SiLU(x) - SiLU(-x) = x
    r = np.random.default_rng(7).standard_normal(4096).astype(np.float32) * 4
    d = oracle.silu(r).astype(np.float64) - oracle.silu(-r).astype(np.float64)
    assert np.all(np.abs(d - r) <= 4 * 2.0 ** -24 * np.abs(r) + 1e-38)
    # tails: -0 (no NaN) far left, identity far right
    far = oracle.silu(np.array([-1000.0, 1000.0, -88.0, 100.0], np.float32))
    assert far[0] == 0.0 and not np.isnan(far[0])
    assert far[1] == 1000.0 and far[3] == 100.0
    assert np.all(np.isfinite(far))


def test_silu_matches_float64_everywhere():
    x = np.linspace(-20, 20, 100001, dtype=np.float32)
    out = oracle.silu(x).astype(np.float64)
    ref = silu64(x.astype(np.float64))
    assert np.all(np.abs(out - ref) <= 4 * 2.0 ** -24 * np.abs(ref) + 1e-40)


# --------------------------------------------------------------------------- rounding
def test_round_bf16_is_nearest_even():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-30).astype(np.float32),
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        # exact ties: bf16 value + half an ulp
        (I.bf16_bits_to_f32(rng.integers(0x3000, 0x5000, 5000, dtype=np.uint16)).view(np.uint32)
         + np.uint32(0x8000)).view(np.float32),
    ])
    r = oracle.round_bf16(x)
    v = bf16_values(r)
    up = bf16_values((r.astype(np.int32) + 1).astype(np.uint16))
    dn = bf16_values((r.astype(np.int32) - 1).astype(np.uint16))
    x64 = x.astype(np.float64)
    err = np.abs(x64 - v)
    # nearest: no neighbour (same sign region) is strictly closer
    assert np.all(err <= np.abs(x64 - up))
    assert np.all(err <= np.abs(x64 - dn))
    # ties go to the even pattern
    tie = (err == np.abs(x64 - up)) | (err == np.abs(x64 - dn))
    tie &= err > 0
    assert tie.sum() >= 4000
    assert np.all((r[tie] & 1) == 0)
    # decode is exact and inverse of encode on bf16 values
    assert np.array_equal(oracle.round_bf16(oracle.decode_bf16(r)), r)


# --------------------------------------------------------------------------- special case A = I
def test_identity_A_gives_elementwise_gate():
    """A = I_K: g = W1, u = W2 exactly, so Y = SiLU(W1) (.) W2 element-wise."""
    K, N = 48, 40
    rng = np.random.default_rng(3)
    a = I.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    w1 = rand_bits(rng, (K, N), 2.0)
    w2 = rand_bits(rng, (K, N), 2.0)
    y, g, u = oracle.swiglu_rows(a, w1, w2, with_gate_up=True)
    assert np.array_equal(g.astype(np.float64), bf16_values(w1))
    assert np.array_equal(u.astype(np.float64), bf16_values(w2))
    ref = silu64(bf16_values(w1)) * bf16_values(w2)
    assert np.all(np.abs(y - ref) <= 4 * 2.0 ** -24 * np.abs(ref) + 1e-38)
    # one-hot rows pick single weight rows
    perm = rng.permutation(K)[:7]
    a1 = I.f32_to_bf16_bits(np.eye(K, dtype=np.float32)[perm])
    y1 = oracle.swiglu(a1, w1, w2)
    assert np.array_equal(y1, y[perm])


# --------------------------------------------------------------------------- invariants
@pytest.fixture(scope="module")
def medium():
    rng = np.random.default_rng(5)
    M, K, N = 37, 72, 56
    return (rand_bits(rng, (M, K)), rand_bits(rng, (K, N), 1 / math.sqrt(K)),
            rand_bits(rng, (K, N), 1 / math.sqrt(K)))


def test_zero_weights_give_zero(medium):
    a, w1, w2 = medium
    z = np.zeros_like(w1)
    assert np.all(oracle.swiglu(a, w1, z) == 0.0)
    assert np.all(oracle.swiglu(a, z, w2) == 0.0)  # SiLU(0) = 0


def test_interleaved_equals_separate_bitwise(medium):
    a, w1, w2 = medium
    wf = oracle.pack_interleaved(w1, w2)
    assert np.array_equal(wf, I.interleave_columns(w1, w2))
    assert np.array_equal(wf[:, 0::2], w1) and np.array_equal(wf[:, 1::2], w2)
    ys = oracle.swiglu(a, w1, w2)
    yi = oracle.swiglu(a, wf, layout=oracle.LAYOUT_INTERLEAVED)
    assert np.array_equal(ys.view(np.uint32), yi.view(np.uint32))
    # swapping the pair roles (Gate odd, Up even) must change the result
    wswap = I.interleave_columns(w2, w1)
    yw = oracle.swiglu(a, wswap, layout=oracle.LAYOUT_INTERLEAVED)
    assert not np.allclose(yw, ys)


def test_permutation_equivariance(medium):
    a, w1, w2 = medium
    rng = np.random.default_rng(9)
    y = oracle.swiglu(a, w1, w2)
    pr = rng.permutation(a.shape[0])
    pc = rng.permutation(w1.shape[1])
    yp = oracle.swiglu(a[pr], w1[:, pc], w2[:, pc])
    assert np.array_equal(yp.view(np.uint32), y[pr][:, pc].view(np.uint32))


def test_power_of_two_scaling_of_up(medium):
    a, w1, w2 = medium
    y = oracle.swiglu(a, w1, w2)
    for k in (-3, 1, 4):
        w2s = I.f32_to_bf16_bits(I.bf16_bits_to_f32(w2) * np.float32(2.0 ** k))
        ys = oracle.swiglu(a, w1, w2s)
        assert np.array_equal(ys, y * np.float32(2.0 ** k))


def test_rows_and_cols_agree_bitwise(medium):
    a, w1, w2 = medium
    y, g, u = oracle.swiglu_rows(a, w1, w2, with_gate_up=True, nthreads=3)
    cols = [0, 5, 17, 55]
    yc, gc, uc = oracle.swiglu_cols(a, w1, w2, cols=cols, with_gate_up=True, nthreads=2)
    assert np.array_equal(yc, y[:, cols]) and np.array_equal(gc, g[:, cols])
    assert np.array_equal(uc, u[:, cols])
    wf = oracle.pack_interleaved(w1, w2)
    yci = oracle.swiglu_cols(a, wf, layout=oracle.LAYOUT_INTERLEAVED, cols=cols)
    assert np.array_equal(yci, y[:, cols])
    rows = [36, 0, 12]
    yr = oracle.swiglu_rows(a, w1, w2, rows=rows)
    assert np.array_equal(yr, y[rows])


def test_thread_count_does_not_change_bits(medium):
    a, w1, w2 = medium
    y1 = oracle.swiglu(a, w1, w2, nthreads=1)
    y7 = oracle.swiglu(a, w1, w2, nthreads=7)
    assert np.array_equal(y1.view(np.uint32), y7.view(np.uint32))


def test_empty_shapes():
    a = np.zeros((0, 8), np.uint16)
    w = np.zeros((8, 16), np.uint16)
    assert oracle.swiglu(a, w, w).shape == (0, 16)
    a = np.zeros((3, 0), np.uint16)
    w = np.zeros((0, 5), np.uint16)
    y = oracle.swiglu(a, w, w)          # empty sums: g = u = 0, y = 0
    assert y.shape == (3, 5) and np.all(y == 0.0)


def test_unfused_emulation_rounds_intermediates(medium):
    a, w1, w2 = medium
    y_emul, gb, ub = oracle.swiglu_unfused_emulation(a, w1, w2)
    _, g, u = oracle.swiglu_rows(a, w1, w2, with_gate_up=True)
    assert np.array_equal(gb, I.f32_to_bf16_bits(g))
    assert np.array_equal(ub, I.f32_to_bf16_bits(u))
    ref = silu64(bf16_values(gb)) * bf16_values(ub)
    assert np.all(np.abs(y_emul - ref) <= 4 * 2.0 ** -24 * np.abs(ref) + 1e-38)


# --------------------------------------------------------------------------- full size vs float64
@pytest.mark.parametrize("wl", I.WORKLOADS, ids=lambda w: w.name)
def test_fullsize_rows_against_float64(wl):
    """Oracle rows at the workloads' real sizes vs a float64 matmul of the same bits.

    The fp32 oracle must sit far inside the parity tolerance (2^-10 absolute
    floor), so that the tolerance budget is spent on the GPU, not here.
    """
    a, w1, w2 = I.workload_inputs(wl)
    rows = np.unique(np.r_[0, wl.M - 1, np.random.default_rng(1).integers(0, wl.M, 6)])
    y = oracle.swiglu_rows(a, w1, w2, rows=rows)
    A64 = bf16_values(a[rows])
    g = A64 @ bf16_values(w1)
    u = A64 @ bf16_values(w2)
    ref = silu64(g) * u
    err = np.abs(y - ref)
    assert err.max() < 2.0 ** -10 / 16, err.max()
    assert np.all(err <= 0.01 * np.abs(ref) / 16 + 2.0 ** -10 / 16)
