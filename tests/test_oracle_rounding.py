"""Pins for the oracle's bf16 and 8-bit-float rounding (CPU only).

bf16 is the pages' compute type (diycv.top, section 关键公式, dtype table).
The pages leave the 8-bit float of the double quantisation unspecified
(section 方法总览 item 3: "8-bit float"); the oracle reads it as OCP E4M3
(E4M3FN). Both encoders are checked against torch's independent CPU
conversions and against hand-derived special values.
"""

import numpy as np
import pytest
import torch

from oracle import nf4


def torch_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_on_random_and_special():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),      # subnormals
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    # exact ties: low 16 bits == 0x8000, with both parities of the kept bit
    bits = rng.integers(0, 2 ** 31, 20000, dtype=np.uint32) & np.uint32(0x7F7F0000)
    ties = (bits | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    np.testing.assert_array_equal(nf4.bf16_rne(x), torch_bf16_bits(x))


def test_bf16_hand_values():
    cases = {
        1.0: 0x3F80,
        1.0 + 2 ** -8: 0x3F80,          # tie, kept mantissa even -> down
        1.0 + 3 * 2 ** -8: 0x3F82,      # tie, kept mantissa odd -> up
        1.0 + 2 ** -8 + 2 ** -20: 0x3F81,
        -2.0: 0xC000,
    }
    for v, b in cases.items():
        assert int(nf4.bf16_rne(np.array([v], np.float32))[0]) == b, v


def test_e4m3_decode_table_facts():
    codes = np.arange(256, dtype=np.uint8)
    vals = nf4.e4m3_decode(codes)
    finite = vals[np.isfinite(vals)]
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert finite.size == 254
    assert np.unique(finite).size == 253                  # +0 and -0 coincide
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0   # largest finite
    assert vals[0x01] == 2.0 ** -9                        # smallest subnormal
    assert vals[0x08] == 2.0 ** -6                        # smallest normal
    assert vals[0x38] == 1.0
    assert np.all(np.diff(vals[:0x7F]) > 0)               # monotone in the code


def test_e4m3_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ov = nf4.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(tv), np.isnan(ov))
    ok = ~np.isnan(ov)
    np.testing.assert_array_equal(tv[ok].astype(np.float64), ov[ok])
    rng = np.random.default_rng(5)
    v = np.concatenate([
        (rng.uniform(-448, 448, 100000)).astype(np.float32),
        (rng.standard_normal(100000) * 0.01).astype(np.float32),
        (rng.standard_normal(10000) * 1e-4).astype(np.float32),
    ])
    tc = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(nf4.e4m3_encode(v), tc)


def test_e4m3_reencode_ties_and_saturation():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = nf4.e4m3_decode(codes).astype(np.float32)
    np.testing.assert_array_equal(nf4.e4m3_encode(vals), codes)
    # midpoint of 1.0 (0x38, even) and 1.125 (0x39) rounds to the even code
    assert nf4.e4m3_encode(np.array([1.0625], np.float32))[0] == 0x38
    # midpoint of 1.125 (0x39) and 1.25 (0x3A) rounds up to the even code
    assert nf4.e4m3_encode(np.array([1.1875], np.float32))[0] == 0x3A
    # saturation instead of NaN
    big = np.array([448.0, 449.0, 500.0, 1e30, -1e30], np.float32)
    np.testing.assert_array_equal(nf4.e4m3_encode(big), [0x7E, 0x7E, 0x7E, 0x7E, 0xFE])
    # below half the smallest subnormal -> zero with the input's sign
    assert nf4.e4m3_encode(np.array([2.0 ** -11], np.float32))[0] == 0x00
    assert nf4.e4m3_encode(np.array([-2.0 ** -11], np.float32))[0] == 0x80


def test_denormals_are_not_flushed():
    # the oracle's fp32 steps rely on IEEE gradual underflow
    tiny = np.float32(2.0 ** -140)
    assert tiny * np.float32(2.0) == np.float32(2.0 ** -139)
    assert np.float32(1.0) / np.float32(2.0 ** 127) == np.float32(2.0 ** -127)
