"""Writes conversion_digests.json: SHA-256 digests of the oracle's fp32 ->
bf16 (round to nearest even) and fp32 -> E4M3 (nearest, ties to the even
code, saturating at +-448) over all 2^32 fp32 bit patterns, in 256 chunks of
2^24 consecutive patterns. The formats are the pages' (diycv.top "QLoRA
论文解读", section 关键公式, the dtype table: first-level constants in an
8-bit float, compute in bf16); the functions are oracle.nf4.bf16_rne and
oracle.nf4.e4m3_encode. Calls nothing but the oracle.

Domain: finite patterns; for bf16 the oracle's own domain, |x| below the
largest finite bf16 (bf16_rne refuses inputs whose upper bf16 neighbour is
infinite, so the 2 x 2^15 patterns from the largest bf16 up to the tie
are left out; the library never meets magnitudes near 3.4e38). Patterns
outside the domain hold 0 in the digested arrays (only chunks 127 and 255
have any).

    python tests/golden/make_conversion_digests.py   # about 2 minutes on 8 cores
"""
import hashlib
import json
import os
import sys
from multiprocessing import Pool

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

CHUNK_LOG2 = 24
NCHUNKS = 1 << (32 - CHUNK_LOG2)
OUT = os.path.join(HERE, "conversion_digests.json")


def patterns(chunk: int) -> np.ndarray:
    return (np.arange(1 << CHUNK_LOG2, dtype=np.uint64) + (chunk << CHUNK_LOG2)).astype(np.uint32)


def domains(p: np.ndarray):
    """(finite, bf16 rounding stays finite) masks of uint32 bit patterns."""
    mag = p & np.uint32(0x7FFFFFFF)
    finite = mag < np.uint32(0x7F800000)
    bf16_ok = mag < np.uint32(0x7F7F0000)
    return finite, bf16_ok


def chunk_digests(chunk: int):
    from oracle import nf4

    p = patterns(chunk)
    x = p.view(np.float32)
    finite, bf16_ok = domains(p)
    bf = np.zeros(p.size, dtype=np.uint16)
    bf[bf16_ok] = nf4.bf16_rne(x[bf16_ok])
    e8 = np.zeros(p.size, dtype=np.uint8)
    e8[finite] = nf4.e4m3_encode(x[finite])
    return chunk, hashlib.sha256(bf.tobytes()).hexdigest(), hashlib.sha256(e8.tobytes()).hexdigest()


def main():
    with Pool(min(8, os.cpu_count() or 1)) as pool:
        res = sorted(pool.map(chunk_digests, range(NCHUNKS)))
    doc = {
        "what": "sha256 of the oracle's conversions over 2^24-pattern chunks of all fp32 bit patterns",
        "chunk_log2": CHUNK_LOG2,
        "bf16_rne_uint16le": [r[1] for r in res],
        "e4m3_encode_uint8": [r[2] for r in res],
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=0)
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
