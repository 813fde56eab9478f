"""Alternative 4-bit data types for the blockwise quantiser (CPU oracle). Test infrastructure only.

The QLoRA pages compare NF4 + DQ with three other 4-bit data types, Int4,
FP4 E2M1 and FP4 E3M0 (page diycv.top "QLoRA 论文解读", section
实验设置与主要结果 item 1, the Pile Common Crawl perplexity table), but
define none of them beyond the name. Each is built here as a 16-entry
ascending table of fp32 values in [-1, 1] (plus, where the format has fewer
than 16 distinct values, one unused entry below -1), so that the same
blockwise absmax scaling, nearest-code rounding, double quantisation and
dequantisation apply unchanged (``oracle.nf4.quantize(w, q)``).

Readings (also listed in the design notes):

* Int4: the pages' Int8 absmax formula X = round(127 / absmax(X) * X)
  (section 方法总览 item 1) with 4-bit signed integers: the levels k / 7,
  k = -7..7, of x = w / absmax. The table holds k / 7 for k = -8..7 in
  index order; k = -8 (index 0, value -8/7) is never produced since
  |x| <= 1. The zero is index 8.
* FP4 E2M1: 1 sign, 2 exponent and 1 mantissa bit with exponent bias 1
  (the OCP microscaling E2M1 element: subnormal 0.5 * m for exponent 0,
  2^(e-1) * (1 + m/2) otherwise), magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6},
  scaled by 1/6 so that the largest is 1 (absmax maps to the top code).
  +0 and -0 are one value, leaving 15 distinct values; index 0 holds the
  unused -2.
* FP4 E3M0: 1 sign, 3 exponent bits, no mantissa. Exponent field 0 encodes
  zero; field e >= 1 encodes 2^e up to a common bias, so after scaling the
  largest to 1 the magnitudes are {0} and 2^-6 .. 2^0. 15 distinct values;
  index 0 holds the unused -2.

Each table value is a float64 quotient rounded once to fp32 (the E3M0
values are powers of two and exact).
"""

from __future__ import annotations

import numpy as np

from . import nf4

_F32 = np.float32
_F64 = np.float64

NAMES = ("nf4", "int4", "fp4_e2m1", "fp4_e3m0")
UNUSED_LOW = -2.0   # index-0 filler of the FP4 tables (never produced)


def e2m1_magnitudes() -> list[float]:
    """All non-negative values of the E2M1 element (bias 1), ascending, deduplicated."""
    vals = set()
    for e in range(4):          # 2 exponent bits
        for m in range(2):      # 1 mantissa bit
            if e == 0:
                vals.add(0.5 * m)                       # subnormal: 2^(1-1) * m/2
            else:
                vals.add(2.0 ** (e - 1) * (1.0 + m / 2.0))
    return sorted(vals)


def e3m0_magnitudes() -> list[float]:
    """Non-negative values of E3M0 with field 0 = zero, up to the common bias."""
    return [0.0] + [2.0 ** e for e in range(1, 8)]


def _signed_table(mags: list[float]) -> np.ndarray:
    top = max(mags)
    pos = [m / top for m in mags if m > 0.0]
    vals = [UNUSED_LOW] + sorted([-p for p in pos]) + [0.0] + pos
    assert len(vals) == 16
    return np.array(vals, dtype=_F64).astype(_F32)


def int4_codebook() -> np.ndarray:
    """k / 7 for k = -8..7 (index = k + 8), each rounded once to fp32."""
    return np.array([k / 7.0 for k in range(-8, 8)], dtype=_F64).astype(_F32)


def fp4_e2m1_codebook() -> np.ndarray:
    return _signed_table(e2m1_magnitudes())


def fp4_e3m0_codebook() -> np.ndarray:
    return _signed_table(e3m0_magnitudes())


def codebook(name: str) -> np.ndarray:
    """The 16-entry fp32 table of a 4-bit data type, ascending."""
    if name == "nf4":
        return nf4.nf4_codebook()
    if name == "int4":
        return int4_codebook()
    if name == "fp4_e2m1":
        return fp4_e2m1_codebook()
    if name == "fp4_e3m0":
        return fp4_e3m0_codebook()
    raise ValueError(f"unknown 4-bit data type {name!r}")


def zero_code(q: np.ndarray) -> int:
    """Index of the table's exact zero (the code of an all-zero block)."""
    z = np.flatnonzero(np.asarray(q, dtype=_F32) == 0.0)
    if z.size != 1:
        raise ValueError("a 4-bit table needs exactly one zero")
    return int(z[0])
