"""NF4 + double-quantisation oracle (CPU, NumPy). Test infrastructure only.

Sources (the QLoRA pages):

* NF4 codebook: page diycv.top "QLoRA 论文解读", section 方法总览 item 2
  ("NF4"), the equation q_i = 1/2 [Q(i/(2^k+1)) + Q((i+1)/(2^k+1))], the
  normalisation to [-1, 1] and the separate construction of the negative and
  positive halves with one exact zero; neura.market analysis, "How It Works"
  (asymmetric so that zero is exact).
* Blockwise quantisation: same page, item 1 (flatten, contiguous blocks of
  size B, one constant per block, absmax scaling as in the Int8 example);
  block size 64 for the base weights.
* Double quantisation: item 3 (first-level constants re-quantised to an
  8-bit float with block size 256; 8/64 + 32/(64*256) = 0.127 bit/param;
  constants are positive, so their mean is subtracted first); neura.market
  "How It Works" (block 256, mean subtraction).
* doubleDequant(c1, c2, W) = dequant(dequant(c1, c2), W): section 关键公式;
  the dtype table there (W in NF4, first-level constants FP8, second-level
  FP32, compute in BF16).

Readings where the pages leave a step open (each is also listed in the
design notes):

* codebook: the quantile formula is used for i >= 1 only (i = 0 needs
  Q(0) = -inf). For an odd count c, S_c = {1/2 [Q(i/(c+2)) + Q((i+1)/(c+2))],
  i = 1..c}; c = 15 gives the pages' denominator 2^4 + 1 = 17. The 7 negative
  members of S_15 are divided by |min S_15|, the 8 positive members of S_17
  by max S_17, and the 16th code is the exact zero. Ascending order.
* nearest code, ties to the lower index; element 2j is the low nibble of
  byte j, element 2j+1 the high nibble; an unused high nibble is 0.
* a block whose absmax is below 2^-126 is a zero block (every code is the
  table's exact zero, 7 for NF4; a := 0). Otherwise x = RN32(w * RN32(1 / a)).
* the DQ mean is one fp32 value per tensor: mu = RN32(S / n) where S is the
  float64 adjacent-pair tree sum of the n block absmax values.
* the 8-bit float is OCP E4M3 ("E4M3FN": bias 7, no infinities, max 448),
  the group absmax of (a - mu) maps to 448, rounding is to nearest even
  after an fp32 quotient, saturating at +-448.
* constant dequant a' = RN32(RN32(e4m3(c) * sigma) + mu) (no fused
  multiply-add); weight dequant w' = bf16_RNE(RN32(q[code] * a')).
"""

from __future__ import annotations

import math
import statistics

import numpy as np

BLOCK = 64          # first-level block size (weights per absmax constant)
DQ_BLOCK = 256      # second-level block size (constants per fp32 scale)
E4M3_MAX = 448.0
FP32_MIN_NORMAL = 2.0 ** -126

_F32 = np.float32
_F64 = np.float64


# --------------------------------------------------------------------------
# NF4 codebook
# --------------------------------------------------------------------------

def normal_quantile(p: float) -> float:
    """Quantile function Q of the standard normal N(0, 1) (library primitive)."""
    return statistics.NormalDist(0.0, 1.0).inv_cdf(p)


def quantile_midpoint_set(c: int, quantile=normal_quantile) -> list[float]:
    """S_c: the pages' q_i midpoints of adjacent N(0,1) quantiles, c of them.

    q_i = 1/2 [Q(i/(c+2)) + Q((i+1)/(c+2))] for i = 1..c. For c = 2^k - 1 the
    denominator is 2^k + 1, the pages' formula (diycv.top, section 方法总览
    item 2). c must be odd; the set is symmetric with an exact middle zero.
    """
    if c % 2 != 1:
        raise ValueError("c must be odd")
    d = c + 2
    vals = []
    for i in range(1, c + 1):
        vals.append(0.5 * (quantile(i / d) + quantile((i + 1) / d)))
    # the middle element is 1/2 [Q(m/d) + Q(1 - m/d)] = 0 in exact arithmetic
    vals[c // 2] = 0.0
    return vals


def nf4_codebook_f64(quantile=normal_quantile) -> np.ndarray:
    """The 16 NF4 values in float64, ascending (before the fp32 rounding)."""
    s15 = quantile_midpoint_set(15, quantile)
    s17 = quantile_midpoint_set(17, quantile)
    neg = [v for v in s15 if v < 0.0]
    pos = [v for v in s17 if v > 0.0]
    neg_scale = -min(s15)
    pos_scale = max(s17)
    neg_n = [v / neg_scale for v in neg]
    pos_n = [v / pos_scale for v in pos]
    vals = sorted(neg_n + [0.0] + pos_n)
    return np.array(vals, dtype=_F64)


def nf4_codebook(quantile=normal_quantile) -> np.ndarray:
    """The 16 NF4 codes as fp32 (each float64 value rounded once, to nearest)."""
    return nf4_codebook_f64(quantile).astype(_F32)


def nf4_midpoints(q: np.ndarray | None = None) -> np.ndarray:
    """Exact midpoints m_j = (q_j + q_{j+1}) / 2, j = 0..14, in float64.

    The q_j are fp32, so their float64 sum and half are exact.
    """
    if q is None:
        q = nf4_codebook()
    q64 = q.astype(_F64)
    return (q64[:-1] + q64[1:]) * 0.5


# --------------------------------------------------------------------------
# bf16 and E4M3 rounding
# --------------------------------------------------------------------------

def f32_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=_F32).view(np.uint32)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(_F32)


CHUNK = 1 << 20   # elementwise passes run over slices of this many elements


def _bf16_rne_slice(x: np.ndarray) -> np.ndarray:
    bits = x.view(np.uint32)
    lo = (bits >> np.uint32(16)).astype(np.uint32)           # toward zero
    hi = lo + np.uint32(1)                                   # away from zero
    lo_v = (lo << np.uint32(16)).view(_F32).astype(_F64)
    hi_v = (hi << np.uint32(16)).view(_F32).astype(_F64)
    if not np.all(np.isfinite(hi_v[np.abs(x) > 0])):
        raise ValueError("bf16_rne: result would overflow")
    xv = x.astype(_F64)
    d_lo = np.abs(xv - lo_v)
    d_hi = np.abs(hi_v - xv)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == 1))
    # exact bf16 values (low 16 bits zero) have d_lo == 0 and keep lo
    return np.where(take_hi, hi, lo).astype(np.uint16)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even mantissa.

    Written as the definition: of the two bf16 neighbours of x (truncation
    towards zero and one bf16 ulp further from zero) take the nearer, and on
    a tie the one whose last mantissa bit is 0. Inputs must be finite and
    must not round beyond the largest finite bf16 value. Elementwise, so it
    is evaluated slice by slice.
    """
    x = np.ascontiguousarray(x, dtype=_F32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_rne: non-finite input")
    flat = x.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint16)
    for i in range(0, flat.size, CHUNK):
        out[i:i + CHUNK] = _bf16_rne_slice(flat[i:i + CHUNK])
    return out.reshape(x.shape)


def e4m3_decode(c: np.ndarray) -> np.ndarray:
    """OCP E4M3 (E4M3FN) code -> value, float64.

    1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
    is subnormal (m * 2^-9); S.1111.111 is NaN; there are no infinities.
    """
    c = np.asarray(c, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


_E4M3_POS_VALUES = e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0x00..0x7E


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp32 value -> E4M3 code: nearest representable, ties to even code,
    saturating at +-448 (never NaN). The sign bit is the sign bit of v."""
    v = np.ascontiguousarray(v, dtype=_F32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    av = np.abs(v.astype(_F64))
    table = _E4M3_POS_VALUES                       # strictly increasing
    hi = np.searchsorted(table, av, side="left")   # first entry >= av
    hi = np.minimum(hi, len(table) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = np.abs(av - table[lo])
    d_hi = np.abs(table[hi] - av)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(av >= E4M3_MAX, 0x7E, code)
    sign = np.signbit(v).astype(np.int64) << 7
    return (code | sign).astype(np.uint8).reshape(v.shape)


# --------------------------------------------------------------------------
# Blockwise NF4 quantisation with double quantisation
# --------------------------------------------------------------------------

def n_blocks(numel: int) -> int:
    return (numel + BLOCK - 1) // BLOCK


def n_groups(numel: int) -> int:
    return (n_blocks(numel) + DQ_BLOCK - 1) // DQ_BLOCK


def tree_sum_f64(v: np.ndarray) -> float:
    """Adjacent-pair tree sum in float64: at each level s'[i] = s[2i] + s[2i+1];
    an odd last element passes through unchanged. Empty input sums to 0."""
    s = np.asarray(v, dtype=_F64).reshape(-1)
    if s.size == 0:
        return 0.0
    while s.size > 1:
        even = s.size - (s.size % 2)
        nxt = s[0:even:2] + s[1:even:2]
        if s.size % 2:
            nxt = np.concatenate([nxt, s[-1:]])
        s = nxt
    return float(s[0])


def block_absmax(flat: np.ndarray) -> np.ndarray:
    """First-level constants: absmax of each contiguous 64-block (exact).
    Blocks whose absmax is below the smallest normal fp32 become 0."""
    nb = n_blocks(flat.size)
    pad = np.zeros(nb * BLOCK, dtype=_F32)
    pad[: flat.size] = flat
    a = np.max(np.abs(pad.reshape(nb, BLOCK)), axis=1).astype(_F32)
    return np.where(a < _F32(FP32_MIN_NORMAL), _F32(0.0), a).astype(_F32)


def nearest_codes(x: np.ndarray, q: np.ndarray) -> np.ndarray:
    """code(x) = number of midpoints m_j strictly below x, which is the index
    of the nearest codebook value with ties going to the lower index."""
    m = nf4_midpoints(q)
    xs = np.asarray(x, dtype=_F32)
    flat = xs.reshape(-1)
    out = np.empty(flat.size, dtype=np.uint8)
    for i in range(0, flat.size, CHUNK):
        x64 = flat[i:i + CHUNK].astype(_F64)
        code = np.zeros(x64.shape, dtype=np.uint8)
        for mj in m:
            code += (x64 > mj)
        out[i:i + CHUNK] = code
    return out.reshape(xs.shape)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Element 2j -> low nibble of byte j, element 2j+1 -> high nibble.
    An odd count leaves the last byte's high nibble at 0."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size % 2:
        c = np.concatenate([c, np.zeros(1, dtype=np.uint8)])
    return (c[0::2] | (c[1::2] << np.uint8(4))).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, numel: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out[:numel]


def quantize(w: np.ndarray, q: np.ndarray | None = None, double_quant: bool = True) -> dict:
    """NF4 blockwise quantisation (B = 64) with double quantisation (B = 256).

    With ``double_quant=False`` the first-level constants are kept as the
    fp32 block absmax (``absmax32``), which is the blockwise quantisation of
    the pages' section 方法总览 item 1 without item 3; the DQ buffers are
    absent.

    ``w`` is the weight in its stored layout (any shape; it is flattened in
    row-major order). fp32 input, or bf16 already widened exactly to fp32.
    Returns a dict with the stored buffers ``codes`` (uint8, packed nibbles),
    ``absmax8`` (uint8 E4M3 codes, one per block), ``scale2`` (fp32, one per
    group of 256 blocks), ``mean`` (fp32, one per tensor) and, for tests,
    the first-level fp32 constants ``absmax`` and the unpacked ``codes4``.
    """
    if q is None:
        q = nf4_codebook()
    flat = np.ascontiguousarray(w, dtype=_F32).reshape(-1)
    if not np.all(np.isfinite(flat)):
        raise ValueError("quantize: non-finite weight")
    numel = flat.size
    nb = n_blocks(numel)
    ng = n_groups(numel)

    # --- first level: absmax per block, normalise, nearest NF4 code --------
    a = block_absmax(flat)
    zero_block = a == 0
    safe_a = np.where(zero_block, _F32(1.0), a)
    r = (_F32(1.0) / safe_a).astype(_F32)                 # RN32(1/a)
    pad = np.zeros(nb * BLOCK, dtype=_F32)
    pad[:numel] = flat
    blocks = pad.reshape(nb, BLOCK)
    codes4 = np.empty((nb, BLOCK), dtype=np.uint8)
    step = CHUNK // BLOCK
    for b0 in range(0, nb, step):
        x = (blocks[b0:b0 + step] * r[b0:b0 + step, None]).astype(_F32)  # RN32(w * r)
        codes4[b0:b0 + step] = nearest_codes(x, q)
    zeros = np.flatnonzero(q == 0.0)
    if zeros.size != 1:
        raise ValueError("quantize: the table needs exactly one zero")
    codes4[zero_block, :] = zeros[0]                       # exact zero code (7 for NF4)
    codes4 = codes4.reshape(-1)[:numel]
    if not double_quant:
        return {"numel": numel, "codes": pack_nibbles(codes4), "absmax32": a, "absmax": a, "codes4": codes4}

    # --- second level: mean-centre, 8-bit float per group of 256 ----------
    mu = _F32(tree_sum_f64(a.astype(_F64)) / nb) if nb else _F32(0.0)
    d = (a - mu).astype(_F32)                               # RN32(a - mu)
    dpad = np.zeros(ng * DQ_BLOCK, dtype=_F32)
    dpad[:nb] = d
    A = np.max(np.abs(dpad.reshape(ng, DQ_BLOCK)), axis=1).astype(_F32)
    sigma = (A / _F32(E4M3_MAX)).astype(_F32)               # RN32(A / 448)
    sigma = np.where(sigma < _F32(FP32_MIN_NORMAL), _F32(0.0), sigma).astype(_F32)
    sig_b = np.repeat(sigma, DQ_BLOCK)[:nb]
    live = sig_b != 0
    v = np.zeros(nb, dtype=_F32)
    v[live] = (d[live] / sig_b[live]).astype(_F32)           # RN32(d / sigma)
    absmax8 = e4m3_encode(v)
    absmax8[~live] = 0

    return {
        "numel": numel,
        "codes": pack_nibbles(codes4),
        "absmax8": absmax8,
        "scale2": sigma.astype(_F32),
        "mean": np.array([mu], dtype=_F32),
        "absmax": a,
        "codes4": codes4,
    }


def dequant_constants(absmax8: np.ndarray, scale2: np.ndarray, mean) -> np.ndarray:
    """dequant(c1, c2): a'_b = RN32(RN32(e4m3(c_b) * sigma_g) + mu), fp32."""
    c = np.asarray(absmax8, dtype=np.uint8)
    nb = c.size
    dec = e4m3_decode(c).astype(_F32)          # every E4M3 value is an fp32
    sig = np.repeat(np.asarray(scale2, dtype=_F32), DQ_BLOCK)[:nb]
    mu = _F32(np.asarray(mean, dtype=_F32).reshape(-1)[0])
    prod = (dec * sig).astype(_F32)
    return (prod + mu).astype(_F32)


def dequantize_f32(qt: dict, q: np.ndarray | None = None) -> np.ndarray:
    """doubleDequant before the bf16 rounding: RN32(q[code] * a'), flat fp32."""
    if q is None:
        q = nf4_codebook()
    numel = qt["numel"]
    codes4 = unpack_nibbles(qt["codes"], numel)
    if "absmax32" in qt:                       # no double quantisation: a' is the block absmax
        ap = np.asarray(qt["absmax32"], dtype=_F32)
    else:
        ap = dequant_constants(qt["absmax8"], qt["scale2"], qt["mean"])
    out = np.empty(numel, dtype=_F32)
    for i in range(0, numel, CHUNK):               # CHUNK is a multiple of BLOCK
        c = codes4[i:i + CHUNK]
        a_e = np.repeat(ap[i // BLOCK:(i + c.size + BLOCK - 1) // BLOCK], BLOCK)[:c.size]
        out[i:i + CHUNK] = (q[c] * a_e).astype(_F32)
    return out


def dequantize(qt: dict, shape=None, q: np.ndarray | None = None) -> np.ndarray:
    """doubleDequant(c1, c2, W) -> bf16 bit patterns (uint16), given shape."""
    out = bf16_rne(dequantize_f32(qt, q))
    return out.reshape(shape) if shape is not None else out


def storage_bits_per_param(numel: int, double_quant: bool = True) -> float:
    """Bits per weight spent on quantisation constants, from buffer sizes.

    With DQ: one E4M3 byte per 64-block plus one fp32 scale per 256 blocks
    plus the per-tensor fp32 mean. Without DQ: one fp32 absmax per block.
    """
    nb = n_blocks(numel)
    ng = n_groups(numel)
    if double_quant:
        return (nb * 8 + ng * 32 + 32) / numel
    return nb * 32 / numel
