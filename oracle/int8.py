"""Blockwise Int8 absmax codec (CPU oracle). Test infrastructure only.

The QLoRA pages introduce blockwise quantisation with the FP32 -> Int8
absmax formula, X_int8 = round(127 / absmax(X) * X), applied per contiguous
block of B elements of the flattened tensor with one constant per block
(page diycv.top "QLoRA 论文解读", section 方法总览 item 1; neura.market
"QLoRA", section "How It Works", blockwise quantisation). This module writes
that formula out, in the pages' order: the scale factor first, then the
product, then the rounding.

Readings (also listed in the design notes):

* The constant stored per block is the fp32 absmax a; the factor is
  c = RN32(127 / a), a correctly rounded fp32 division, and the code is
  round(RN32(x * c)) with ties to even, clamped to [-127, 127]. The pages
  leave the rounding of ties and the arithmetic precision open.
* A block whose absmax is below 2^-120 (all zeros, or so small that 127 / a
  would leave the fp32 range) is a zero block: every code is 0.
* Dequantisation inverts the factor: x' = RN32(code * RN32(a / 127)), one
  correctly rounded division per block and one product per element, as
  fp32, or rounded once more to bf16 (round to nearest even).
* Blocks cut the row-major flattening; the last block may be short (the
  padding zeros never change an absmax and produce no codes).
"""

from __future__ import annotations

import numpy as np

from . import nf4

_F32 = np.float32
ZERO_BLOCK_BELOW = np.float32(2.0 ** -120)


def n_blocks(numel: int, block: int) -> int:
    return -(-numel // block)


def block_absmax(flat: np.ndarray, block: int) -> np.ndarray:
    """max |x| of each block of the flattened fp32 tensor (exact)."""
    nb = n_blocks(flat.size, block)
    pad = np.zeros(nb * block, _F32)
    pad[: flat.size] = flat
    return np.abs(pad.reshape(nb, block)).max(axis=1)


def quantize(x: np.ndarray, block: int = 64) -> dict:
    """Int8 codes and fp32 block absmax of ``x`` (fp32 values; a bf16 tensor
    is passed widened to fp32). Returns {"codes": int8[numel], "absmax":
    f32[nb], "block": block}."""
    flat = np.ascontiguousarray(x, dtype=_F32).reshape(-1)
    if not np.all(np.isfinite(flat)):
        raise ValueError("inputs must be finite")
    a = block_absmax(flat, block)
    zero = a < ZERO_BLOCK_BELOW
    with np.errstate(divide="ignore"):
        c = np.where(zero, _F32(0), _F32(127) / np.where(zero, _F32(1), a)).astype(_F32)   # RN32(127/a)
    per_elem = np.repeat(c, block)[: flat.size]
    v = (flat * per_elem).astype(_F32)                    # RN32(x * c)
    codes = np.clip(np.rint(v), -127, 127).astype(np.int8)   # ties to even
    return {"codes": codes, "absmax": a, "block": block}


def dequantize_f32(qt: dict) -> np.ndarray:
    """x' = RN32(code * RN32(a / 127)) for every element (flat fp32)."""
    codes, a, block = qt["codes"], qt["absmax"], qt["block"]
    d = (a.astype(_F32) / _F32(127)).astype(_F32)        # RN32(a / 127)
    per_elem = np.repeat(d, block)[: codes.size]
    return (codes.astype(_F32) * per_elem).astype(_F32)


def dequantize_bf16(qt: dict) -> np.ndarray:
    """The fp32 result rounded to bf16 (round to nearest even), as uint16 bits."""
    return nf4.bf16_rne(dequantize_f32(qt))
