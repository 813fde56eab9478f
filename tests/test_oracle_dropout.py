"""Pins of the LoRA-dropout oracle (oracle/dropout.py): Philox4x32-10 against
its published known-answer vectors (tests/golden/philox4x32_10_kat.json),
the keep rate and its independence across elements and seeds, the scaling
of kept elements (exact where 1/(1-p) is a power of two), p = 0 reducing to
the layer without dropout, and the backward pass as the exact adjoint of
the forward in X, L1 and L2 for a fixed mask.
"""

import json
import os

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import dropout, linear, nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answers():
    for v in json.load(open(GOLDEN))["vectors"]:
        ctr = [int(x, 16) for x in v["counter"]]
        key = [int(x, 16) for x in v["key"]]
        got = dropout.philox4x32_10(ctr, key).tolist()
        assert got == [int(x, 16) for x in v["output"]]


def test_counter_layout_and_words():
    # element e uses counter (e/4, 0, 0, 0) under key (lo, hi) of the seed and word e % 4
    seed = 0x0123456789ABCDEF
    w = dropout.words(10, seed)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    b0 = dropout.philox4x32_10([0, 0, 0, 0], key)
    b2 = dropout.philox4x32_10([2, 0, 0, 0], key)
    assert w[:4].tolist() == b0.tolist() and w[8:10].tolist() == b2[:2].tolist()


@pytest.mark.parametrize("p", [0.1, 0.05])
def test_keep_rate_and_independence(p):
    M, K = 1024, 4096
    keep = dropout.keep_mask(M, K, p, seed=7)
    n = keep.size
    rate = keep.mean()
    assert abs(rate - (1 - p)) < 5 * np.sqrt(p * (1 - p) / n)
    # neighbouring elements (same counter block and across blocks) are uncorrelated
    a, b = keep[:, :-1].astype(np.float64), keep[:, 1:].astype(np.float64)
    corr = np.corrcoef(a.ravel(), b.ravel())[0, 1]
    assert abs(corr) < 5 / np.sqrt(n)
    # another seed gives another mask with the same rate
    other = dropout.keep_mask(M, K, p, seed=8)
    assert 0.0 < np.mean(keep != other) < 2.5 * p


def test_threshold_and_scale():
    assert dropout.threshold(0.0) == 0
    assert dropout.threshold(0.5) == 2 ** 31
    assert dropout.keep_scale(0.5) == np.float32(2.0)
    assert dropout.keep_scale(0.0) == np.float32(1.0)
    with pytest.raises(ValueError):
        dropout.threshold(1.0)


def test_kept_values_are_scaled_inputs():
    rng = np.random.default_rng(3)
    X = workloads.to_bf16_bits(rng.standard_normal((64, 256)).astype(np.float32))
    # p = 0.5: the factor is exactly 2, so kept values are exactly 2 x
    Xd = dropout.drop_input(X, 0.5, seed=11)
    keep = dropout.keep_mask(64, 256, 0.5, 11)
    xf = nf4.bf16_bits_to_f32(X)
    np.testing.assert_array_equal(nf4.bf16_bits_to_f32(Xd)[keep], 2 * xf[keep])
    assert np.all(Xd[~keep] == 0)
    # p = 0.1: within one bf16 rounding of x / 0.9
    Xd = nf4.bf16_bits_to_f32(dropout.drop_input(X, 0.1, seed=11)).astype(np.float64)
    keep = dropout.keep_mask(64, 256, 0.1, 11)
    want = xf.astype(np.float64) / 0.9
    assert np.all(np.abs(Xd[keep] - want[keep]) <= 2.0 ** -8 * np.abs(want[keep]) + 1e-30)
    # p = 0: the input itself
    np.testing.assert_array_equal(dropout.drop_input(X, 0.0, seed=11), X)


def layer(seed=5, M=12, K=128, N=40, r=8):
    rng = np.random.default_rng(seed)
    inp = workloads.draw_linear(rng, workloads.LinearShape("t", K, N), M, r, 0.5, "normal", 0.02, True)
    Wd = nf4.dequantize(nf4.quantize(inp.W), inp.W.shape)
    return inp, Wd


def test_p_zero_is_the_plain_layer():
    inp, Wd = layer()
    Y0, T0 = linear.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s)
    Y1, T1 = dropout.linear_fwd(inp.X, Wd, inp.L1, inp.L2, inp.s, 0.0, 9)
    np.testing.assert_array_equal(Y0, Y1)
    np.testing.assert_array_equal(T0, T1)
    for a, b in zip(linear.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY),
                    dropout.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY, 0.0, 9)):
        np.testing.assert_array_equal(a, b)


def test_backward_is_the_adjoint_of_the_forward():
    # with p = 0.5 the dropped input is exactly 2 x keep, so for a fixed mask
    # the forward is linear in X, in L1 and in L2, and the backward must be
    # its exact adjoint: <dY, Y(V)> = <dX, V>, and likewise for the adapters
    inp, Wd = layer()
    p, seed = 0.5, 13
    M, K = inp.X.shape
    rng = np.random.default_rng(21)
    dX, dL1, dL2 = dropout.linear_bwd(inp.X, Wd, inp.L1, inp.L2, inp.s, inp.dY, p, seed)
    dYf = linear.widen(inp.dY)
    V = workloads.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    YV, _ = dropout.linear_fwd(V, Wd, inp.L1, inp.L2, inp.s, p, seed)
    assert np.isclose(np.sum(dYf * YV), np.sum(dX * linear.widen(V)), rtol=1e-10, atol=1e-12)
    Xd = linear.widen(dropout.drop_input(inp.X, p, seed))
    V1 = rng.standard_normal(inp.L1.shape)
    lhs = np.sum(dYf * (inp.s * (Xd @ V1) @ linear.widen(inp.L2)))
    assert np.isclose(lhs, np.sum(dL1 * V1), rtol=1e-10, atol=1e-12)
    V2 = rng.standard_normal(inp.L2.shape)
    lhs = np.sum(dYf * (inp.s * (Xd @ linear.widen(inp.L1)) @ V2))
    assert np.isclose(lhs, np.sum(dL2 * V2), rtol=1e-10, atol=1e-12)
    # and the mask really reaches dX: dropped positions get only the base term
    keep = dropout.keep_mask(M, K, p, seed)
    base = dYf @ linear.widen(Wd)
    np.testing.assert_allclose(dX[~keep], base[~keep], rtol=0, atol=1e-12)
    assert np.max(np.abs(dX[keep] - base[keep])) > 1e-6
