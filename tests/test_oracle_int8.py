"""Pins of the Int8 absmax codec oracle (oracle/int8.py) against values fixed
by the formula X_int8 = round(127 / absmax(X) * X) of the QLoRA pages
(diycv.top, section 方法总览 item 1) and by arithmetic: hand-worked blocks,
exhaustive search for the nearest integer, sign symmetry, power-of-two
scale invariance, the worst-case round-trip bound, zero blocks, ragged tails
and the blockwise-versus-per-tensor outlier effect the passage motivates.
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads
from oracle import int8


def test_hand_worked_block_with_unit_factor():
    # absmax 127 gives the factor 127/127 = 1 exactly, so the codes are the
    # inputs rounded to the nearest integer, ties to even
    x = np.zeros(64, np.float32)
    x[:9] = [127.0, 2.5, 3.5, -2.5, 0.5, 1.5, 126.5, -0.49, 100.25]
    qt = int8.quantize(x)
    assert qt["absmax"].tolist() == [127.0]
    assert qt["codes"][:9].tolist() == [127, 2, 4, -2, 0, 2, 126, 0, 100]
    assert not qt["codes"][9:].any()
    # the inverse factor is 127/127 = 1: dequantisation returns the codes
    assert int8.dequantize_f32(qt)[:9].tolist() == [127.0, 2.0, 4.0, -2.0, 0.0, 2.0, 126.0, 0.0, 100.0]


def test_hand_worked_block_with_absmax_one():
    x = np.zeros(64, np.float32)
    x[:5] = [1.0, -0.5, 0.25, 0.75, -1.0]       # 127 x = 127, -63.5, 31.75, 95.25, -127
    qt = int8.quantize(x)
    assert qt["codes"][:5].tolist() == [127, -64, 32, 95, -127]
    d = np.float32(1.0) / np.float32(127.0)
    assert int8.dequantize_f32(qt)[:2].tolist() == [np.float32(127 * d), np.float32(-64 * d)]


@pytest.mark.parametrize("block", [64, 256, 4096])
def test_codes_are_the_nearest_integer_by_exhaustive_search(block):
    rng = np.random.default_rng(5)
    x = workloads.random_weight(rng, 3 * block + 17, "student-t4")
    qt = int8.quantize(x, block)
    a = int8.block_absmax(x, block)
    ks = np.arange(-127, 128, dtype=np.float64)
    for b in range(a.size):
        c = np.float32(127.0) / a[b]
        seg = x[b * block:(b + 1) * block]
        for j, xv in enumerate(seg):
            v = float(np.float32(np.float64(xv) * np.float64(c)))     # one fp32 rounding of the product
            dist = np.abs(ks - v)
            best = ks[dist == dist.min()]
            want = best[0] if best.size == 1 else best[np.abs(best) % 2 == 0][0]   # tie: the even one
            assert qt["codes"][b * block + j] == want


def test_absmax_element_takes_the_extreme_code_and_signs_are_symmetric():
    rng = np.random.default_rng(6)
    x = workloads.random_weight(rng, 64 * 50, "normal")
    qt = int8.quantize(x)
    blocks = x.reshape(50, 64)
    codes = qt["codes"].reshape(50, 64)
    idx = np.abs(blocks).argmax(axis=1)
    ext = codes[np.arange(50), idx]
    assert np.all(np.abs(ext) == 127)
    assert np.all(np.sign(ext) == np.sign(blocks[np.arange(50), idx]))
    neg = int8.quantize(-x)
    np.testing.assert_array_equal(neg["codes"], -qt["codes"])
    np.testing.assert_array_equal(neg["absmax"], qt["absmax"])


@pytest.mark.parametrize("k", [-20, -3, 1, 7])
def test_power_of_two_scaling_changes_only_the_constant(k):
    rng = np.random.default_rng(7)
    x = workloads.random_weight(rng, 64 * 40 + 5, "normal")
    qt = int8.quantize(x)
    qs = int8.quantize((x * np.float32(2.0 ** k)).astype(np.float32))
    np.testing.assert_array_equal(qs["codes"], qt["codes"])
    np.testing.assert_array_equal(qs["absmax"], (qt["absmax"] * np.float32(2.0 ** k)).astype(np.float32))


@pytest.mark.parametrize("block", [64, 1024])
def test_round_trip_error_within_half_a_step(block):
    # |x - x'| <= a/254 (half the code spacing) plus a few fp32 roundings
    rng = np.random.default_rng(8)
    x = workloads.random_weight(rng, 20 * block + 3, "student-t4")
    qt = int8.quantize(x, block)
    xd = int8.dequantize_f32(qt).astype(np.float64)
    a = np.repeat(qt["absmax"].astype(np.float64), block)[: x.size]
    err = np.abs(x.astype(np.float64) - xd)
    assert np.all(err <= a / 254.0 * (1 + 2.0 ** -20) + 4 * 2.0 ** -24 * a)
    # and the bound is nearly reached somewhere (the codes really are 8-bit)
    assert err.max() > 0.4 * (a / 254.0).max()


def test_zero_and_tiny_blocks():
    x = np.zeros(64 * 4 + 9, np.float32)
    x[64] = np.float32(2.0 ** -121)       # below the zero-block limit
    x[128] = np.float32(2.0 ** -120)      # at the limit: an ordinary block
    x[129] = np.float32(-2.0 ** -121)
    x[192 + 3] = np.float32(0.5)
    x[256 + 8] = np.float32(-3.0)         # the short last block
    qt = int8.quantize(x)
    assert qt["absmax"].tolist() == [0.0, 2.0 ** -121, 2.0 ** -120, 0.5, 3.0]
    c = qt["codes"]
    assert not c[:128].any()
    assert c[128] == 127 and c[129] == -64          # -0.5 * 127 = -63.5 -> -64
    assert c[195] == 127 and c[264] == -127 and c.size == x.size
    assert np.all(int8.dequantize_f32(qt)[:128] == 0.0)


def test_blocks_contain_outliers_that_a_single_scale_spreads():
    # one outlier in the tensor crushes every other value into a few codes when
    # the whole tensor shares one absmax; blocks of 64 confine it to its block
    rng = np.random.default_rng(9)
    x = rng.standard_normal(64 * 256).astype(np.float32)
    x[1000] = 2000.0
    per_tensor = int8.quantize(x, x.size)
    blockwise = int8.quantize(x, 64)
    assert np.mean(np.abs(per_tensor["codes"]) <= 1) > 0.99
    e_t = np.sqrt(np.mean((int8.dequantize_f32(per_tensor) - x) ** 2))
    e_b = np.sqrt(np.mean((int8.dequantize_f32(blockwise) - x) ** 2))
    assert e_b < e_t / 10          # only the outlier's own block loses its small values


def test_bf16_output_is_the_fp32_result_rounded():
    qt = int8.quantize(np.array([1.0, 0.3, -0.7] + [0.0] * 61, np.float32))
    bits = int8.dequantize_bf16(qt)
    f = int8.dequantize_f32(qt)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.abs(back - f) <= np.abs(f) * 2.0 ** -8)


def test_non_finite_input_is_rejected():
    with pytest.raises(ValueError):
        int8.quantize(np.array([1.0, np.inf], np.float32))
