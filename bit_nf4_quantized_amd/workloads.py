"""Seeded synthetic inputs for the QLoRA NF4 hot path.

This module only draws random numbers and arranges them in the shapes of the
workloads; it holds none of the method's arithmetic. Both the oracle-side
tests and the GPU path take their inputs from here, so the two sides always
see the same bytes.

All draws use numpy's PCG64 ``default_rng(seed)`` in a fixed order. Weights
are fp32 in the stored [N][K] (out x in) layout. bf16 tensors are fp32 draws
rounded to bf16 by torch's CPU conversion (round to nearest even) and
returned as uint16 bit patterns.

The QLoRA pages finetune LLaMA 7B-65B on instruction data, which is not
available here; these tensors stand in for them by shape and value
distribution only (N(0, sigma) weights, optionally with a sprinkle of
outliers or heavy Student-t tails; N(0, 1) activations and gradients;
small N(0, 0.01) adapters).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16) via torch's CPU conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


@dataclass(frozen=True)
class LinearShape:
    name: str
    K: int   # in_features
    N: int   # out_features


# LLaMA-shaped 7-linear sets: q, k, v, o, gate, up, down (in x out = K x N).
def llama_linears(hidden: int, ffn: int) -> list[LinearShape]:
    return [
        LinearShape("q", hidden, hidden),
        LinearShape("k", hidden, hidden),
        LinearShape("v", hidden, hidden),
        LinearShape("o", hidden, hidden),
        LinearShape("gate", hidden, ffn),
        LinearShape("up", hidden, ffn),
        LinearShape("down", ffn, hidden),
    ]


LLAMA7B = llama_linears(4096, 11008)
LLAMA33B = llama_linears(6656, 17920)
LLAMA65B = llama_linears(8192, 22016)

# Named workloads (sizes as used by the tests and the benchmark).
WORKLOADS = {
    "tiny-512": dict(seed=1, linears=[LinearShape("w", 512, 512)], M=64, r=8, s=2.0,
                     w_kind="normal", w_std=0.02),
    "llama7b-layer": dict(seed=2, linears=LLAMA7B, M=8192, r=64, s=0.25,
                          w_kind="normal+outliers", w_std=0.02),
    "gemv": dict(seed=3, linears=[LinearShape("up", 4096, 11008),
                                  LinearShape("down", 11008, 4096)],
                 M_list=(1, 4, 16), r=64, s=0.25, w_kind="normal", w_std=0.02),
    "llama65b-quantize": dict(seed=4, linears=LLAMA65B, layers=80,
                              w_kind="normal", w_std=0.015),
    "llama33b-layer": dict(seed=5, linears=LLAMA33B, M=8192, r=64, s=0.25,
                           w_kind="student-t4", w_std=0.02),
}


def draw_weight(rng: np.random.Generator, N: int, K: int, kind: str, std: float) -> np.ndarray:
    """Frozen base weight, fp32 [N][K]."""
    if kind in ("normal", "normal+outliers"):
        w = (std * rng.standard_normal((N, K), dtype=np.float32)).astype(np.float32)
        if kind == "normal+outliers":
            # 0.1 % of the entries, at distinct positions, scaled by 10
            n_out = int(round(0.001 * N * K))
            pos = rng.choice(N * K, size=n_out, replace=False)
            flat = w.reshape(-1)
            flat[pos] *= np.float32(10.0)
        return w
    if kind == "student-t4":
        return (std / np.sqrt(2.0) * student_t4(rng, (N, K))).astype(np.float32)
    raise ValueError(kind)


def student_t4(rng: np.random.Generator, shape) -> np.ndarray:
    """Student-t draws with 4 degrees of freedom (variance 2), float64.

    t = Z / sqrt(C / 4) with Z ~ N(0, 1) and C ~ chi-square(4); C is the
    sum of two independent Exp(1) draws times 2, so t = Z sqrt(2 / (E1 + E2)).
    This is the textbook construction of the t distribution, drawn here from
    three fast float32 streams (Z, E1, E2 in that order) instead of numpy's
    gamma-based standard_t.
    """
    z = rng.standard_normal(shape, dtype=np.float32).astype(np.float64)
    e1 = rng.standard_exponential(shape, dtype=np.float32).astype(np.float64)
    e2 = rng.standard_exponential(shape, dtype=np.float32).astype(np.float64)
    return z * np.sqrt(2.0 / (e1 + e2))


@dataclass
class LinearInputs:
    W: np.ndarray        # fp32 [N][K]
    L1: np.ndarray       # bf16 bits [K][r]
    L2: np.ndarray       # bf16 bits [r][N]
    X: np.ndarray        # bf16 bits [M][K]
    dY: np.ndarray       # bf16 bits [M][N] (None for forward-only workloads)
    s: float


def draw_linear(rng: np.random.Generator, shape: LinearShape, M: int, r: int, s: float,
                w_kind: str, w_std: float, with_grad: bool = True) -> LinearInputs:
    """One linear's inputs, drawn in the order W, L1, L2, X, dY."""
    W = draw_weight(rng, shape.N, shape.K, w_kind, w_std)
    L1 = to_bf16_bits(0.01 * rng.standard_normal((shape.K, r), dtype=np.float32))
    L2 = to_bf16_bits(0.01 * rng.standard_normal((r, shape.N), dtype=np.float32))
    X = to_bf16_bits(rng.standard_normal((M, shape.K), dtype=np.float32))
    dY = to_bf16_bits(rng.standard_normal((M, shape.N), dtype=np.float32)) if with_grad else None
    return LinearInputs(W=W, L1=L1, L2=L2, X=X, dY=dY, s=s)


def tiny_512() -> LinearInputs:
    """512x512 fp32 weight N(0, 0.02); 64 tokens; r = 8, s = 2 (seed 1)."""
    cfg = WORKLOADS["tiny-512"]
    rng = np.random.default_rng(cfg["seed"])
    return draw_linear(rng, cfg["linears"][0], cfg["M"], cfg["r"], cfg["s"],
                       cfg["w_kind"], cfg["w_std"])


def layer_linear(name: str, index: int, M: int | None = None, with_grad: bool = True):
    """Inputs of linear ``index`` (0..6: q, k, v, o, gate, up, down) of a
    7-linear layer set. Each linear has its own stream
    default_rng([seed, index]), drawn in the order W, L1, L2, X, dY, so any
    linear can be drawn alone. ``M`` may shrink the token count for tests."""
    cfg = WORKLOADS[name]
    shp = cfg["linears"][index]
    rng = np.random.default_rng([cfg["seed"], index])
    M = cfg["M"] if M is None else M
    return shp, draw_linear(rng, shp, M, cfg["r"], cfg["s"], cfg["w_kind"], cfg["w_std"], with_grad)


def layer_weight(name: str, index: int) -> np.ndarray:
    """Only the fp32 weight of linear ``index`` (the first draw of its stream)."""
    cfg = WORKLOADS[name]
    shp = cfg["linears"][index]
    rng = np.random.default_rng([cfg["seed"], index])
    return draw_weight(rng, shp.N, shp.K, cfg["w_kind"], cfg["w_std"])


def gemv_inputs(K: int, N: int, M: int, seed: int = 3, r: int = 64, s: float = 0.25) -> LinearInputs:
    """Small-M decode-style forward: W [N][K] N(0, 0.02), X [M][K]."""
    rng = np.random.default_rng([seed, K, N, M])
    return draw_linear(rng, LinearShape("gemv", K, N), M, r, s, "normal", 0.02, with_grad=False)


def quantize_weight(shape: LinearShape, seed: int, index: int, std: float = 0.015) -> np.ndarray:
    """A single fp32 weight for quantize-throughput runs, seeded per tensor."""
    rng = np.random.default_rng([seed, index])
    return draw_weight(rng, shape.N, shape.K, "normal", std)


def random_weight(rng: np.random.Generator, numel: int, kind: str = "normal", std: float = 0.02) -> np.ndarray:
    """Flat fp32 weight of any length (ragged tails, short blocks and groups)."""
    if kind == "normal":
        return (std * rng.standard_normal(numel, dtype=np.float32)).astype(np.float32)
    if kind == "student-t4":
        return (std / np.sqrt(2.0) * student_t4(rng, numel)).astype(np.float32)
    raise ValueError(kind)
