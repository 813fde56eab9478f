"""Adapter merge into the 16-bit dequantised base (CPU oracle). Test infrastructure only.

The pages warn that folding the trained adapters back into the 4-bit base
(W + B A re-quantised) loses the adapters' precision, and that the merge
belongs in the dequantised 16-bit base, or the adapters stay separate
(robocikowo.com "QLoRA", the list of common mistakes, the entry on merging
the adapters; diycv.top "QLoRA 论文解读",
section 训练与推理流程, inference keeps the 4-bit base and the adapters).
In this layout (base stored as Wt[N][K], Y = X Wt^T + s (X L1) L2) the
merged weight is

    M[n][k] = Wd[n][k] + s * sum_j L1[k][j] L2[j][n]

with Wd the doubleDequant bf16 weight, so that X M^T is the layer's forward
product. Readings (also in the design notes): the base term is the bf16
dequantised value (the "16-bit dequantised base"); the adapter term and the
sum are exact here (float64, library matmul), and the result is rounded
once to bf16, to nearest with ties to even.
"""

from __future__ import annotations

import numpy as np

from .linear import widen
from .nf4 import bf16_rne

_F64 = np.float64
_F32 = np.float32


def merge_exact(Wd_bits, L1, L2, s: float) -> np.ndarray:
    """Wd + s (L1 L2)^T in float64 (Wd, L1, L2 as bf16 bits or float arrays)."""
    Wd = widen(Wd_bits)
    delta = widen(L1) @ widen(L2)            # [K][N]
    return Wd + _F64(s) * delta.T


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest, ties to even, in one rounding.

    Narrowing to fp32 first with round-to-odd (truncate, then force the last
    bit to 1 if anything was dropped) keeps 16 guard bits beyond bf16's 8, so
    the following fp32 -> bf16 round-to-nearest-even is the correct rounding
    of the float64 value."""
    x = np.asarray(x, dtype=_F64)
    t = x.astype(_F32)
    over = np.abs(t.astype(_F64)) > np.abs(x)
    t = np.where(over, np.nextafter(t, _F32(0)), t).astype(_F32)       # toward zero
    inexact = t.astype(_F64) != x
    bits = t.view(np.uint32) | inexact.astype(np.uint32)
    return bf16_rne(bits.view(_F32))


def merge(Wd_bits, L1, L2, s: float) -> np.ndarray:
    """The merged weight as bf16 bits [N][K]."""
    return f64_to_bf16_rne(merge_exact(Wd_bits, L1, L2, s))
