"""QLoRA linear layer oracle (CPU, NumPy, float64). Test infrastructure only.

Sources (the QLoRA pages):

* forward: Y = X W + s X L1 L2 with L1 in R^{h x r}, L2 in R^{r x o}
  (diycv.top "QLoRA 论文解读", section 问题背景, LoRA equation); with the
  base weight replaced by doubleDequant(c1, c2, W_NF4) in BF16 (section
  关键公式, equation for Y^BF16). The scale s is kept as in the LoRA
  equation (the 关键公式 rendering omits it).
* backward: gradients flow through the dequantised BF16 base weight to the
  layer input, and only the adapters get parameter gradients; there is no
  weight gradient (section 关键公式, text after the dtype table; training
  steps 4-5; neura.market analysis, "How It Works").

Layout used here and by the library: the base weight is stored as
Wt[N][K] (out_features x in_features), the transpose of the pages' W; so
Y = X Wt^T + s (X L1) L2 and dX = dY Wt + s (dY L2^T) L1^T.

Inputs arrive as bf16 bit patterns (uint16) and are widened exactly; every
product and sum is then taken in float64 with library matmuls, so the result
is the exact layer up to float64 rounding. No dropout (reading: the pages'
LoRA dropout is a training-recipe setting, not part of the layer).
"""

from __future__ import annotations

import numpy as np

from .nf4 import bf16_bits_to_f32, bf16_rne

_F64 = np.float64


def widen(bits_or_array) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 exactly; float arrays pass through."""
    a = np.asarray(bits_or_array)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(_F64)
    return a.astype(_F64)


def linear_fwd(X, Wt, L1, L2, s: float):
    """Y = X Wt^T + s (X L1) L2 in float64. Returns (Y, T) with T = X L1."""
    X, Wt, L1, L2 = widen(X), widen(Wt), widen(L1), widen(L2)
    T = X @ L1
    Y = X @ Wt.T + float(s) * (T @ L2)
    return Y, T


def linear_bwd(X, Wt, L1, L2, s: float, dY):
    """Gradients of the layer for upstream gradient dY, float64.

    dX  = dY Wt + s (dY L2^T) L1^T      (through the frozen base and the adapter)
    dL1 = s X^T (dY L2^T)
    dL2 = s (X L1)^T dY
    There is no gradient for the frozen base weight.
    """
    X, Wt, L1, L2, dY = widen(X), widen(Wt), widen(L1), widen(L2), widen(dY)
    s = float(s)
    U = dY @ L2.T
    T = X @ L1
    dX = dY @ Wt + s * (U @ L1.T)
    dL1 = s * (X.T @ U)
    dL2 = s * (T.T @ dY)
    return dX, dL1, dL2


def linear_fwd_rows(X, Wt, L1, L2, s: float, rows):
    """Selected rows of Y (for sampled checks at full size)."""
    X = widen(np.asarray(X)[rows])
    Y, _ = linear_fwd(X, Wt, L1, L2, s)
    return Y


def linear_bwd_dx_rows(Wt, L1, L2, s: float, dY, rows):
    """Selected rows of dX (row m of dX depends on row m of dY only)."""
    dY = widen(np.asarray(dY)[rows])
    Wt, L1, L2 = widen(Wt), widen(L1), widen(L2)
    return dY @ Wt + float(s) * ((dY @ L2.T) @ L1.T)


def bf16_floor(R) -> float:
    """The error that rounding the exact result to bf16 alone leaves:
    max |bf16_RNE(R) - R| / RMS(R) (R rounded to fp32 first, then to bf16).
    A bf16 output cannot score below this on the agreement metric."""
    R = np.asarray(R, dtype=_F64)
    rb = widen(bf16_rne(R.astype(np.float32)))
    return rel_err(rb, R)


def bf16_half_ulp(R) -> np.ndarray:
    """Half the spacing of bf16 values in the binade of |R| (8 significand
    bits: values in [2^e, 2^(e+1)) are 2^(e-7) apart), elementwise; below
    the normal range the subnormal spacing 2^-133."""
    a = np.abs(np.asarray(R, dtype=_F64))
    _, e = np.frexp(a)                  # a = f 2^e with f in [0.5, 1): binade exponent e - 1
    e = np.maximum(e - 1, -126)
    return np.where(a > 0, np.ldexp(1.0, e - 8), np.ldexp(1.0, -134))


def rel_err_beyond_bf16(G, R) -> float:
    """The agreement metric for a bf16 output with its own output rounding
    taken out: max over elements of max(0, |G - R| - half a bf16 ulp at R),
    over RMS(R). A correctly rounded bf16 result scores 0; anything the
    computation adds beyond the final rounding (operand or accumulation
    error, a wrong term) counts in full."""
    G = widen(G)
    R = np.asarray(R, dtype=_F64)
    rms = float(np.sqrt(np.mean(R * R))) if R.size else 0.0
    ex = np.maximum(np.abs(G - R) - bf16_half_ulp(R), 0.0)
    top = float(np.max(ex)) if ex.size else 0.0
    return top / rms if rms > 0 else top


def rel_err(G, R) -> float:
    """max |G - R| / RMS(R), G widened to float64; R the oracle result."""
    G = widen(G)
    R = np.asarray(R, dtype=_F64)
    rms = float(np.sqrt(np.mean(R * R)))
    if rms == 0.0:
        return float(np.max(np.abs(G - R))) if G.size else 0.0
    return float(np.max(np.abs(G - R))) / rms
