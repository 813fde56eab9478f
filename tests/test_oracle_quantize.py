"""Pins for the oracle's NF4 quantisation, double quantisation and dequant.

Checked against what the pages fix and against brute force:
* bit accounting printed on diycv.top, section 方法总览 item 3
  (0.5 -> 0.127 bit/param, saving 0.373, about 3 GB at 65B);
* nearest-code quantisation by exhaustive exact search (fractions.Fraction)
  on small tensors, including constructed exact ties;
* special cases: zero blocks, a single block, two blocks, short last block
  and short last group;
* the round-trip error bound implied by the steps;
* the mean-centring of the first-level constants (same item 3; neura.market,
  "How It Works").
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4
from bit_nf4_quantized_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dq_accounting.json")
Q = nf4.nf4_codebook()


def brute_force_codes(w: np.ndarray) -> np.ndarray:
    """Nearest NF4 code of every element by exhaustive exact search.

    Normalisation as the method states it: x = RN32(w * RN32(1/absmax)) per
    64-block; then argmin_j |x - q_j| over Fractions, ties to the lower j.
    """
    flat = np.asarray(w, np.float32).reshape(-1)
    qf = [Fraction(float(v)) for v in Q]
    out = []
    for b0 in range(0, flat.size, 64):
        blk = flat[b0:b0 + 64]
        a = np.float32(max(abs(float(v)) for v in blk))
        if a < np.float32(2.0 ** -126):
            out.extend([7] * blk.size)
            continue
        r = np.float32(1.0) / a
        for v in blk:
            x = Fraction(float(np.float32(v * r)))
            dists = [abs(x - qj) for qj in qf]
            best = min(dists)
            out.append(dists.index(best))        # first index = lower on ties
    return np.array(out, np.uint8)


@pytest.mark.parametrize("numel,kind", [(64, "normal"), (640, "normal"), (1000, "normal"),
                                        (777, "student-t4"), (64 * 3 + 5, "normal")])
def test_codes_match_brute_force(numel, kind):
    rng = np.random.default_rng(numel)
    w = workloads.random_weight(rng, numel, kind)
    qt = nf4.quantize(w)
    np.testing.assert_array_equal(qt["codes4"], brute_force_codes(w))


def test_constructed_ties_go_to_lower_code():
    m = nf4.nf4_midpoints(Q)
    exact = [j for j in range(15) if float(np.float32(m[j])) == m[j]]
    assert exact == [4, 5, 6, 7, 9, 10, 11, 12, 14]
    # block absmax 1.0 makes r = 1 and x = w exactly
    w = np.zeros(64, np.float32)
    w[0] = 1.0
    for i, j in enumerate(exact):
        w[1 + i] = np.float32(m[j])
    # fp32 neighbours of the non-representable midpoints straddle them
    k = 1 + len(exact)
    for j in [0, 1, 2, 3, 8, 13]:
        f = np.float32(m[j])
        below = np.nextafter(f, np.float32(-2)) if f > m[j] else f
        above = np.nextafter(below, np.float32(2))
        assert below < m[j] < above
        w[k], w[k + 1] = below, above
        k += 2
    qt = nf4.quantize(w)
    c = qt["codes4"]
    assert c[0] == 15
    for i, j in enumerate(exact):
        assert c[1 + i] == j, (j, c[1 + i])
    k = 1 + len(exact)
    for j in [0, 1, 2, 3, 8, 13]:
        assert (c[k], c[k + 1]) == (j, j + 1)
        k += 2
    np.testing.assert_array_equal(c, brute_force_codes(w))


def test_end_codes_and_zero_block():
    w = np.zeros(128, np.float32)
    w[64:] = np.linspace(-0.3, 0.2, 64, dtype=np.float32)
    qt = nf4.quantize(w)
    c = qt["codes4"]
    assert np.all(c[:64] == 7) and qt["absmax"][0] == 0
    assert c[64] == 0                     # the element equal to -absmax
    assert c[64 + np.argmax(w[64:])] != 15  # 0.2 < absmax 0.3
    w2 = w.copy()
    w2[64] = 0.3
    assert nf4.quantize(w2)["codes4"][64] == 15
    # subnormal absmax is a zero block too
    w3 = np.full(64, 1e-39, np.float32)
    qt3 = nf4.quantize(w3)
    assert np.all(qt3["codes4"] == 7) and qt3["absmax"][0] == 0


def test_nibble_packing_order():
    codes = np.array([1, 2, 3], np.uint8)
    np.testing.assert_array_equal(nf4.pack_nibbles(codes), [0x21, 0x03])
    np.testing.assert_array_equal(nf4.unpack_nibbles(np.array([0x21, 0x03], np.uint8), 3), codes)


def test_single_block_tensor():
    rng = np.random.default_rng(3)
    w = workloads.random_weight(rng, 64)
    qt = nf4.quantize(w)
    a = np.float32(np.max(np.abs(w)))
    assert qt["mean"][0] == a                       # mu of one constant
    assert qt["scale2"][0] == 0 and qt["absmax8"][0] == 0
    ap = nf4.dequant_constants(qt["absmax8"], qt["scale2"], qt["mean"])
    assert ap[0] == a                               # a' = a exactly


def test_two_block_tensor():
    w = np.zeros(128, np.float32)
    w[5] = 0.5
    w[70] = -0.125
    qt = nf4.quantize(w)
    a0, a1 = np.float32(0.5), np.float32(0.125)
    mu = np.float32((float(a0) + float(a1)) / 2)     # hand value 0.3125
    assert qt["mean"][0] == mu == np.float32(0.3125)
    # d = +-0.1875, group absmax 0.1875 maps to +-448
    assert qt["scale2"][0] == np.float32(0.1875) / np.float32(448)
    assert qt["absmax8"].tolist() == [0x7E, 0xFE]
    ap = nf4.dequant_constants(qt["absmax8"], qt["scale2"], qt["mean"])
    np.testing.assert_allclose(ap, [0.5, 0.125], rtol=2e-7)


def test_tree_sum_pairing_hand_example():
    e = 2.0 ** -53
    # adjacent pairs: (1 + e) -> 1.0 (tie to even), (e + e) = 2e; 1 + 2e exact
    assert nf4.tree_sum_f64(np.array([1.0, e, e, e])) == 1.0 + 2 * e
    # odd element passes through: ((1 + e) + e) -> 1.0, tree gives 1.0
    assert nf4.tree_sum_f64(np.array([1.0, e, e])) == 1.0
    # sequential left-to-right on [e, e, 1] also gives 1 + 2e; tree: (2e) + 1
    assert nf4.tree_sum_f64(np.array([e, e, 1.0])) == 1.0 + 2 * e
    assert nf4.tree_sum_f64(np.array([])) == 0.0
    rng = np.random.default_rng(0)
    v = rng.random(1001)
    exact = sum(Fraction(float(x)) for x in v)
    assert abs(Fraction(nf4.tree_sum_f64(v)) - exact) <= Fraction(11 * 2 ** -53) * sum(Fraction(float(x)) for x in v)


def test_mean_centring():
    rng = np.random.default_rng(9)
    w = workloads.random_weight(rng, 64 * 1000 + 17)
    qt = nf4.quantize(w)
    a = qt["absmax"].astype(np.float64)
    mu = float(qt["mean"][0])
    # mu is the fp32 rounding of the mean of the constants
    assert abs(mu - a.mean()) <= 2.0 ** -24 * abs(a.mean()) + 1e-15
    assert abs(np.sum(a - mu)) <= a.size * 2.0 ** -24 * abs(mu)


def test_bit_accounting_matches_pages():
    with open(GOLDEN) as f:
        g = json.load(f)
    assert nf4.BLOCK == g["block"] and nf4.DQ_BLOCK == g["dq_block"]
    for shp in workloads.LLAMA7B + workloads.LLAMA33B + workloads.LLAMA65B:
        numel = shp.N * shp.K
        with_dq = nf4.storage_bits_per_param(numel, True) - 32 / numel   # without the one mean
        without = nf4.storage_bits_per_param(numel, False)
        assert with_dq == 8 / 64 + 32 / (64 * 256) == 0.126953125
        assert without == g["bits_per_param_without_dq"]
        d = g["printed_decimals"]
        assert round(with_dq, d) == g["bits_per_param_with_dq_printed"]
        assert round(without - with_dq, d) == g["saving_bits_per_param_printed"]
    saving_bytes = g["model_params_65b"] * (0.5 - 0.126953125) / 8
    assert abs(saving_bytes / g["saving_bytes_65b_printed"] - 1) < g["saving_bytes_relative_tolerance"]
    # the stored buffers have exactly these sizes
    qt = nf4.quantize(np.ones(4096 * 64, np.float32))
    assert qt["codes"].nbytes * 8 == 4 * 4096 * 64
    assert qt["absmax8"].nbytes == 4096 and qt["scale2"].nbytes == 4 * 16


@pytest.mark.parametrize("numel,kind", [(64 * 300 + 33, "normal"), (64 * 257, "student-t4"),
                                        (4096 * 4, "normal")])
def test_roundtrip_bound(numel, kind):
    """|w - w'| <= a*h(code) + |q|*|a - a'| + 1/2 ulp_bf16(w') + 2^-24 |q a'|,
    with h the half-gap around the chosen code and |a - a'| bounded by the
    E4M3 step of the scaled constant plus the fp32 roundings."""
    rng = np.random.default_rng(numel)
    w = workloads.random_weight(rng, numel, kind)
    qt = nf4.quantize(w)
    wd = nf4.bf16_bits_to_f32(nf4.dequantize(qt)).astype(np.float64)
    a = np.repeat(qt["absmax"], 64)[:numel].astype(np.float64)
    ap = np.repeat(nf4.dequant_constants(qt["absmax8"], qt["scale2"], qt["mean"]), 64)[:numel].astype(np.float64)
    c = qt["codes4"]
    q64 = Q.astype(np.float64)
    gaps = np.diff(q64)
    h = np.maximum(np.concatenate([[0], gaps])[c], np.concatenate([gaps, [0]])[c]) / 2
    sig = np.repeat(qt["scale2"], 64 * 256)[:numel].astype(np.float64)
    v = np.abs(nf4.e4m3_decode(np.repeat(qt["absmax8"], 64)[:numel]))
    e4m3_half_step = np.where(v < 2 ** -6, 2.0 ** -10, 2.0 ** (np.floor(np.log2(np.maximum(v, 2 ** -6))) - 4))
    da = sig * e4m3_half_step * 1.0001 + 2.0 ** -23 * (np.abs(ap) + abs(float(qt["mean"][0])))
    assert np.all(np.abs(a - ap) <= da + 1e-30)
    ulp_half = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(wd), 2 ** -126))) - 8)
    bound = a * h + np.abs(q64[c]) * da + ulp_half + 2.0 ** -24 * np.abs(q64[c] * ap)
    assert np.all(np.abs(w.astype(np.float64) - wd) <= bound * (1 + 1e-9) + 1e-30)


def test_all_zero_and_exact_code_tensors():
    z = nf4.quantize(np.zeros(1000, np.float32))
    assert np.all(nf4.dequantize(z) == 0)
    assert z["mean"][0] == 0 and np.all(z["scale2"] == 0)
    # a single block of exact codes times a: dequant gives bf16(RN32(q_j a))
    a = np.float32(0.037)
    w = (np.tile(Q, 4) * a).astype(np.float32)
    qt = nf4.quantize(w)
    np.testing.assert_array_equal(qt["codes4"], np.tile(np.arange(16, dtype=np.uint8), 4))
    np.testing.assert_array_equal(nf4.dequantize(qt), nf4.bf16_rne(w))


def test_ragged_sizes_and_buffers():
    for numel in [1, 2, 63, 65, 64 * 256 + 1, 64 * 256 * 2 + 100]:
        rng = np.random.default_rng(numel)
        w = workloads.random_weight(rng, numel)
        qt = nf4.quantize(w)
        nb = -(-numel // 64)
        ng = -(-nb // 256)
        assert qt["codes"].size == -(-numel // 2)
        assert qt["absmax8"].size == nb and qt["scale2"].size == ng
        if numel % 2:
            assert qt["codes"][-1] >> 4 == 0            # unused high nibble
        wd = nf4.bf16_bits_to_f32(nf4.dequantize(qt))
        assert wd.size == numel
        assert np.max(np.abs(wd - w)) <= 0.2 * np.max(np.abs(w)) + 1e-30
