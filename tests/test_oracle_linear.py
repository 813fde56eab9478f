"""Pins for the oracle's QLoRA linear forward and backward (CPU only).

The layer is Y = X W + s X L1 L2 (diycv.top, section 问题背景, LoRA
equation; section 关键公式) with gradients for X, L1 and L2 but none for the
frozen base (text after the dtype table). Checked against pure-Python loops
on tiny shapes, against exact special cases (L2 = 0, W = 0, s = 0), against
the adjoint and Euler identities of a bilinear map, and against central
finite differences in float64.
"""

import numpy as np
import pytest

from oracle import linear, nf4
from bit_nf4_quantized_amd import workloads


def rand_bf16(rng, shape, scale=1.0):
    return workloads.to_bf16_bits(scale * rng.standard_normal(shape).astype(np.float32))


def tiny(rng, M=3, K=5, N=4, r=2):
    return (rand_bf16(rng, (M, K)), rand_bf16(rng, (N, K), 0.3), rand_bf16(rng, (K, r), 0.5),
            rand_bf16(rng, (r, N), 0.5), rand_bf16(rng, (M, N)))


def loops_fwd(X, Wt, L1, L2, s):
    M, K = len(X), len(X[0])
    N = len(Wt)
    r = len(L1[0])
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += X[m][k] * Wt[n][k]
            lora = 0.0
            for j in range(r):
                t = 0.0
                for k in range(K):
                    t += X[m][k] * L1[k][j]
                lora += t * L2[j][n]
            Y[m][n] = acc + s * lora
    return np.array(Y)


def loops_bwd(X, Wt, L1, L2, s, dY):
    M, K = len(X), len(X[0])
    N = len(Wt)
    r = len(L1[0])
    U = [[sum(dY[m][n] * L2[j][n] for n in range(N)) for j in range(r)] for m in range(M)]
    T = [[sum(X[m][k] * L1[k][j] for k in range(K)) for j in range(r)] for m in range(M)]
    dX = [[sum(dY[m][n] * Wt[n][k] for n in range(N)) + s * sum(U[m][j] * L1[k][j] for j in range(r))
           for k in range(K)] for m in range(M)]
    dL1 = [[s * sum(X[m][k] * U[m][j] for m in range(M)) for j in range(r)] for k in range(K)]
    dL2 = [[s * sum(T[m][j] * dY[m][n] for m in range(M)) for n in range(N)] for j in range(r)]
    return np.array(dX), np.array(dL1), np.array(dL2)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_python_loops(seed):
    rng = np.random.default_rng(seed)
    X, Wt, L1, L2, dY = tiny(rng)
    s = 0.75
    w = [linear.widen(a).tolist() for a in (X, Wt, L1, L2, dY)]
    Y, _ = linear.linear_fwd(X, Wt, L1, L2, s)
    np.testing.assert_allclose(Y, loops_fwd(*w[:4], s), rtol=1e-12, atol=1e-14)
    dX, dL1, dL2 = linear.linear_bwd(X, Wt, L1, L2, s, dY)
    lX, lL1, lL2 = loops_bwd(*w[:4], s, w[4])
    np.testing.assert_allclose(dX, lX, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dL1, lL1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dL2, lL2, rtol=1e-12, atol=1e-14)


def test_special_cases():
    rng = np.random.default_rng(7)
    X, Wt, L1, L2, dY = tiny(rng, M=6, K=8, N=5, r=3)
    Xf, Wf, L1f, L2f, dYf = (linear.widen(a) for a in (X, Wt, L1, L2, dY))
    zero_L2 = np.zeros_like(L2)
    Y, _ = linear.linear_fwd(X, Wt, L1, zero_L2, 2.0)
    np.testing.assert_array_equal(Y, Xf @ Wf.T)
    dX, dL1, dL2 = linear.linear_bwd(X, Wt, L1, zero_L2, 2.0, dY)
    np.testing.assert_array_equal(dL1, 0)
    np.testing.assert_allclose(dX, dYf @ Wf, rtol=1e-15)
    np.testing.assert_allclose(dL2, 2.0 * (Xf @ L1f).T @ dYf, rtol=1e-15)
    Y0, _ = linear.linear_fwd(X, np.zeros_like(Wt), L1, L2, 0.5)
    np.testing.assert_allclose(Y0, 0.5 * (Xf @ L1f) @ L2f, rtol=1e-15)
    Ys, _ = linear.linear_fwd(X, Wt, L1, L2, 0.0)
    np.testing.assert_array_equal(Ys, Xf @ Wf.T)
    _, gL1, gL2 = linear.linear_bwd(X, Wt, L1, L2, 0.0, dY)
    assert not np.any(gL1) and not np.any(gL2)


def test_adjoint_and_euler_identities():
    rng = np.random.default_rng(8)
    X, Wt, L1, L2, dY = tiny(rng, M=16, K=32, N=24, r=4)
    s = 0.25
    Xf, L1f, L2f, dYf = (linear.widen(a) for a in (X, L1, L2, dY))
    Y, T = linear.linear_fwd(X, Wt, L1, L2, s)
    dX, dL1, dL2 = linear.linear_bwd(X, Wt, L1, L2, s, dY)
    # Y is linear in X: <dY, Y> = <dX, X>
    assert np.vdot(dYf, Y) == pytest.approx(np.vdot(dX, Xf), rel=1e-12)
    # the LoRA term is linear in L1 and in L2 separately
    lora = s * (Xf @ L1f) @ L2f
    e = np.vdot(dYf, lora)
    assert np.vdot(dL1, L1f) == pytest.approx(e, rel=1e-12)
    assert np.vdot(dL2, L2f) == pytest.approx(e, rel=1e-12)


def test_finite_differences():
    rng = np.random.default_rng(9)
    X, Wt, L1, L2, dY = tiny(rng, M=4, K=6, N=5, r=2)
    s = 1.5
    Xf, Wf, L1f, L2f, dYf = (linear.widen(a) for a in (X, Wt, L1, L2, dY))
    dX, dL1, dL2 = linear.linear_bwd(X, Wt, L1, L2, s, dY)

    def loss(Xv, L1v, L2v):
        Y, _ = linear.linear_fwd(Xv, Wf, L1v, L2v, s)
        return float(np.vdot(dYf, Y))

    h = 1e-4
    for (arr, grad, idx) in [(Xf, dX, (1, 2)), (Xf, dX, (3, 0)), (L1f, dL1, (4, 1)),
                             (L1f, dL1, (0, 0)), (L2f, dL2, (1, 3)), (L2f, dL2, (0, 4))]:
        plus, minus = arr.copy(), arr.copy()
        plus[idx] += h
        minus[idx] -= h
        args_p = [plus if arr is a else a for a in (Xf, L1f, L2f)]
        args_m = [minus if arr is a else a for a in (Xf, L1f, L2f)]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert fd == pytest.approx(grad[idx], rel=1e-7, abs=1e-10)


def test_rel_err_metric():
    R = np.array([3.0, -4.0])          # RMS = sqrt(12.5)
    G = np.array([3.1, -4.0])
    assert linear.rel_err(G, R) == pytest.approx(0.1 / np.sqrt(12.5))
    bf = nf4.bf16_rne(np.array([1.0 + 2 ** -7 + 2 ** -9], np.float32))
    assert linear.rel_err(bf, np.array([1.0 + 2 ** -7 + 2 ** -9])) > 0


@pytest.mark.parametrize("seed", [3, 4])
def test_row_helpers_match_python_loops(seed):
    """The sampled-row helpers give exactly the selected rows of Y and dX,
    checked against the pure-Python loops (a dropped LoRA term, a transposed
    operand or a row mix-up in either helper fails here)."""
    rng = np.random.default_rng(seed)
    X, Wt, L1, L2, dY = tiny(rng, M=7, K=6, N=5, r=3)
    s = 0.5
    w = [linear.widen(a).tolist() for a in (X, Wt, L1, L2, dY)]
    rows = np.array([0, 3, 6])
    lY = loops_fwd(*w[:4], s)
    lX, _, _ = loops_bwd(*w[:4], s, w[4])
    np.testing.assert_allclose(linear.linear_fwd_rows(X, Wt, L1, L2, s, rows), lY[rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(linear.linear_bwd_dx_rows(Wt, L1, L2, s, dY, rows), lX[rows], rtol=1e-12, atol=1e-14)
    # and they agree with the full-tensor functions row for row
    Y, _ = linear.linear_fwd(X, Wt, L1, L2, s)
    dX, _, _ = linear.linear_bwd(X, Wt, L1, L2, s, dY)
    np.testing.assert_allclose(linear.linear_fwd_rows(X, Wt, L1, L2, s, rows), Y[rows], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(linear.linear_bwd_dx_rows(Wt, L1, L2, s, dY, rows), dX[rows], rtol=1e-14, atol=1e-15)


def test_bf16_floor():
    """The output-rounding floor: max |bf16_RNE(R) - R| / RMS(R)."""
    R = np.array([1.0, -1.0, 1.0 + 2 ** -9])       # RMS ~ 1; the third value rounds by 2^-9
    assert linear.bf16_floor(R) == pytest.approx(2 ** -9 / np.sqrt(np.mean(R * R)))
    assert linear.bf16_floor(np.array([0.5, 0.25])) == 0.0


def test_error_beyond_bf16_rounding():
    """A correctly rounded bf16 output scores 0, even where half an ulp is
    far above 2 % of the RMS; one ulp off at the largest element scores half
    an ulp; an error added before the rounding counts in full."""
    rng = np.random.default_rng(11)
    R = rng.standard_normal(4096) * 1.3
    R[7] = 9.71875                                 # a bf16 midpoint in [8, 16): half an ulp (2^-5) away
    rounded = nf4.bf16_rne(R.astype(np.float32))
    assert linear.rel_err_beyond_bf16(rounded, R) == 0.0
    assert linear.rel_err(rounded, R) > 0.015     # the plain metric sees the rounding
    rms = np.sqrt(np.mean(R * R))
    off = rounded.copy()
    off[7] = off[7] + 1                            # next bf16 above: 9.75 -> 9.8125 (RNE picked 9.75)
    got = linear.rel_err_beyond_bf16(off, R)
    expect = (abs(linear.widen(off)[7] - R[7]) - 2.0 ** -5) / rms
    assert got == pytest.approx(expect, rel=1e-12) and got > 0
    shifted = nf4.bf16_rne((R + 0.05 * rms).astype(np.float32))   # a bias before rounding
    assert linear.rel_err_beyond_bf16(shifted, R) > 0.03
    # half ulps: 1.0 -> 2^-8, 9.7 -> 2^-5, 0.3 -> 2^-10, 2^-130 (subnormal) -> 2^-134
    np.testing.assert_array_equal(linear.bf16_half_ulp(np.array([1.0, -9.7, 0.3, 2.0 ** -130])),
                                  [2.0 ** -8, 2.0 ** -5, 2.0 ** -10, 2.0 ** -134])
