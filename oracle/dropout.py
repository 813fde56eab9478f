"""LoRA dropout on the adapter branch (CPU oracle). Test infrastructure only.

The pages' Guanaco settings use LoRA dropout 0.1 for the 7B/13B models and
0.05 for 33B/65B (page diycv.top "QLoRA 论文解读", section 训练与推理流程,
the common settings after the training steps). They do not say where the
dropout sits; the reading here is the usual LoRA one, on the adapter
branch's input: the layer becomes

    Y = X Wd^T + s (Xd L1) L2,    Xd = drop(X)

with Wd the doubleDequant weight. The mask is drawn from Philox4x32-10, the
counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel Random
Numbers: As Easy as 1, 2, 3", SC 2011), written here from that definition:

* state: four 32-bit counter words and two 32-bit key words; ten rounds,
  each (c0, c1, c2, c3) -> (hi(B c2) ^ c1 ^ k0, lo(B c2), hi(A c0) ^ c3 ^ k1,
  lo(A c0)) with A = 0xD2511F53, B = 0xCD9E8D57 and 32 x 32 -> 64-bit
  products, the key bumped by (0x9E3779B9, 0xBB67AE85) after every round;
* element e of the row-major [M][K] input uses counter (lo(e/4), hi(e/4),
  0, 0), key (lo(seed), hi(seed)), and output word e % 4 as u;
* the element is kept iff u >= floor(p 2^32).

Readings (also in the design notes): a kept element is bf16_RNE(RN32(x c))
with c = RN32(1 / (1 - p)) (the adapter product takes bf16 operands, so the
dropped input is a bf16 tensor), a dropped one is +0. In the backward the
rounding of x c is taken as the identity, so the gradient through the
dropout is keep * c: dX = dY Wd + keep * c * (s (dY L2^T) L1^T), dL1 = s
Xd^T (dY L2^T), dL2 = s (Xd L1)^T dY.
"""

from __future__ import annotations

import numpy as np

from .linear import widen
from .nf4 import bf16_bits_to_f32, bf16_rne

_U32 = np.uint64(0xFFFFFFFF)
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85


def philox4x32_10(counter, key) -> np.ndarray:
    """Philox4x32-10 of counters [..., 4] (uint32) under key [2] (or [..., 2]);
    returns [..., 4] uint32."""
    c = np.asarray(counter, dtype=np.uint64) & _U32
    k = np.broadcast_to(np.asarray(key, dtype=np.uint64) & _U32, c.shape[:-1] + (2,))
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = k[..., 0].copy(), k[..., 1].copy()
    for rnd in range(10):
        p0 = np.uint64(PHILOX_M0) * c0           # < 2^64: exact in uint64
        p1 = np.uint64(PHILOX_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _U32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _U32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        if rnd < 9:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _U32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _U32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def threshold(p: float) -> int:
    """floor(p 2^32) for the keep test u >= threshold (0 <= p < 1)."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return int(np.floor(np.float64(np.float32(p)) * 4294967296.0))


def keep_scale(p: float) -> np.float32:
    """c = RN32(1 / (1 - p)) for the fp32 probability p."""
    return np.float32(1.0 / (1.0 - np.float64(np.float32(p))))


def words(numel: int, seed: int) -> np.ndarray:
    """u for elements 0 .. numel-1 (uint32)."""
    n4 = -(-numel // 4)
    idx = np.arange(n4, dtype=np.uint64)
    ctr = np.stack([idx & _U32, idx >> np.uint64(32), np.zeros_like(idx), np.zeros_like(idx)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    return philox4x32_10(ctr, key).reshape(-1)[:numel]


def keep_mask(M: int, K: int, p: float, seed: int) -> np.ndarray:
    """bool [M][K]: True where the element of the row-major input is kept."""
    return (words(M * K, seed) >= np.uint32(threshold(p))).reshape(M, K) if M * K else np.zeros((M, K), bool)


def drop_input(X_bits: np.ndarray, p: float, seed: int) -> np.ndarray:
    """The dropped adapter input Xd as bf16 bits [M][K]."""
    M, K = X_bits.shape
    keep = keep_mask(M, K, p, seed)
    scaled = bf16_rne((bf16_bits_to_f32(X_bits) * keep_scale(p)).astype(np.float32))
    return np.where(keep, scaled, np.uint16(0)).astype(np.uint16)


def linear_fwd(X, Wt, L1, L2, s: float, p: float, seed: int):
    """Y = X Wt^T + s (Xd L1) L2 in float64; returns (Y, T = Xd L1)."""
    Xd = widen(drop_input(np.asarray(X), p, seed))
    T = Xd @ widen(L1)
    Y = widen(X) @ widen(Wt).T + float(s) * (T @ widen(L2))
    return Y, T


def linear_bwd(X, Wt, L1, L2, s: float, dY, p: float, seed: int):
    """(dX, dL1, dL2) of the layer with dropout, float64."""
    X = np.asarray(X)
    M, K = X.shape
    keep = keep_mask(M, K, p, seed)
    Xd = widen(drop_input(X, p, seed))
    dYf, L1f, L2f = widen(dY), widen(L1), widen(L2)
    U = dYf @ L2f.T
    c = np.float64(keep_scale(p))
    dX = dYf @ widen(Wt) + np.where(keep, c, 0.0) * (float(s) * (U @ L1f.T))
    dL1 = float(s) * (Xd.T @ U)
    dL2 = float(s) * ((Xd @ L1f).T @ dYf)
    return dX, dL1, dL2
