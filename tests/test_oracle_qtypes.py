"""Pins for the oracle's alternative 4-bit data types (Int4, FP4 E2M1, FP4 E3M0).

The pages name these types and compare them with NF4 + DQ (diycv.top,
section 实验设置与主要结果 item 1) without defining them; the readings are in
oracle/qtypes.py. Checked here against what fixes them independently of the
oracle's own construction:
* the published E2M1 element values {0, 0.5, 1, 1.5, 2, 3, 4, 6} and the
  E3M0 powers of two, written out literally;
* Int4 as the pages' Int8 absmax formula at 4 bits: the code of x is
  round(7 x) + 8, checked against numpy's rounding away from ties;
* nearest-code rounding of every table by exhaustive exact search
  (fractions.Fraction) on small tensors, ties to the lower index;
* zero blocks take the table's exact zero;
* the pages' reason for NF4: on normally distributed weights it has the
  smallest quantisation error of the four types.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4, qtypes
from bit_nf4_quantized_amd import workloads

TYPES = ["nf4", "int4", "fp4_e2m1", "fp4_e3m0"]


def test_e2m1_table_is_the_published_element_set():
    vals = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]            # OCP E2M1 magnitudes besides 0
    want = [-2.0] + [-v / 6.0 for v in reversed(vals)] + [0.0] + [v / 6.0 for v in vals]
    got = qtypes.codebook("fp4_e2m1")
    np.testing.assert_array_equal(got.view(np.uint32), np.array(want, np.float64).astype(np.float32).view(np.uint32))


def test_e3m0_table_is_powers_of_two():
    want = [-2.0] + [-(2.0 ** -k) for k in range(0, 7)] + [0.0] + [2.0 ** -k for k in range(6, -1, -1)]
    got = qtypes.codebook("fp4_e3m0")
    np.testing.assert_array_equal(got, np.array(want, np.float32))


def test_int4_codes_are_int8_style_rounding():
    # X^Int4 = round(7 / absmax(X) * X): the code of x in [-1, 1] is round(7 x) + 8
    rng = np.random.default_rng(7)
    x = rng.uniform(-1.0, 1.0, 20000).astype(np.float32)
    frac = np.abs(7.0 * x.astype(np.float64) - np.floor(7.0 * x.astype(np.float64)) - 0.5)
    x = x[frac > 1e-6]                                     # away from exact ties
    code = nf4.nearest_codes(x, qtypes.codebook("int4")).astype(np.int64)
    np.testing.assert_array_equal(code - 8, np.rint(7.0 * x.astype(np.float64)).astype(np.int64))


@pytest.mark.parametrize("name", TYPES)
def test_tables_are_well_formed(name):
    q = qtypes.codebook(name)
    assert q.dtype == np.float32 and q.size == 16
    assert np.all(np.diff(q.astype(np.float64)) > 0)
    assert np.count_nonzero(q == 0.0) == 1
    assert q[15] == 1.0
    # the extreme normalised inputs reach the +-1 entries; entry 0 is -1 or unreachable below it
    ends = nf4.nearest_codes(np.array([-1.0, 1.0], np.float32), q)
    assert q[ends[0]] == -1.0 and q[ends[1]] == 1.0
    if name != "nf4":
        assert q[0] < -1.0 and ends[0] == 1


@pytest.mark.parametrize("name", TYPES)
@pytest.mark.parametrize("numel,kind", [(640, "normal"), (777, "student-t4")])
def test_codes_match_brute_force(name, numel, kind):
    q = qtypes.codebook(name)
    rng = np.random.default_rng(numel + len(name))
    w = workloads.random_weight(rng, numel, kind)
    qt = nf4.quantize(w, q)
    qf = [Fraction(float(v)) for v in q]
    want = []
    for b0 in range(0, numel, 64):
        blk = w[b0:b0 + 64]
        a = np.float32(max(abs(float(v)) for v in blk))
        r = np.float32(1.0) / a
        for v in blk:
            x = Fraction(float(np.float32(v * r)))
            d = [abs(x - qj) for qj in qf]
            want.append(d.index(min(d)))
    np.testing.assert_array_equal(qt["codes4"], np.array(want, np.uint8))


@pytest.mark.parametrize("name", TYPES)
def test_zero_block_takes_the_zero_code(name):
    q = qtypes.codebook(name)
    w = np.zeros(3 * 64, np.float32)
    w[64:128] = np.linspace(-1.0, 1.0, 64, dtype=np.float32)
    qt = nf4.quantize(w, q)
    z = qtypes.zero_code(q)
    assert np.all(qt["codes4"][:64] == z) and np.all(qt["codes4"][128:] == z)
    assert np.all(nf4.dequantize_f32(qt, q)[:64] == 0.0)


def test_nf4_has_the_smallest_error_on_normal_weights():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal(1 << 16) * 0.02).astype(np.float32)
    err = {}
    for name in TYPES:
        q = qtypes.codebook(name)
        d = nf4.dequantize_f32(nf4.quantize(w, q), q).astype(np.float64)
        err[name] = np.sqrt(np.mean((d - w) ** 2) / np.mean(w.astype(np.float64) ** 2))
    assert min(err, key=err.get) == "nf4", err


# ---- without double quantisation --------------------------------------------------------

@pytest.mark.parametrize("name", ["nf4", "int4"])
def test_no_dq_keeps_the_exact_block_absmax(name):
    q = qtypes.codebook(name)
    rng = np.random.default_rng(21)
    w = workloads.random_weight(rng, 64 * 37 + 9, "normal")
    qt = nf4.quantize(w, q, double_quant=False)
    pad = np.zeros(64 * 38, np.float32)
    pad[: w.size] = w
    a = np.abs(pad.reshape(38, 64)).max(axis=1)
    np.testing.assert_array_equal(qt["absmax32"], a)
    assert "absmax8" not in qt
    codes = nf4.unpack_nibbles(qt["codes"], w.size)
    want = (q[codes] * np.repeat(a, 64)[: w.size]).astype(np.float32)
    np.testing.assert_array_equal(nf4.dequantize_f32(qt, q), want)
    # the codes are those of the DQ path (the first level is the same)
    np.testing.assert_array_equal(qt["codes"], nf4.quantize(w, q)["codes"])


def test_dq_constant_error_is_within_the_e4m3_step():
    # a' - a comes from one E4M3 rounding of (a - mu) / sigma (3 mantissa bits:
    # relative error <= 2^-4) plus fp32 roundings
    rng = np.random.default_rng(22)
    w = workloads.random_weight(rng, 64 * 4096, "student-t4")
    qt = nf4.quantize(w)
    a = qt["absmax"].astype(np.float64)
    ap = nf4.dequant_constants(qt["absmax8"], qt["scale2"], qt["mean"]).astype(np.float64)
    mu = float(qt["mean"][0])
    assert np.all(np.abs(ap - a) <= 2.0 ** -4 * np.abs(a - mu) + 2.0 ** -20 * np.abs(a)), np.max(np.abs(ap - a))
