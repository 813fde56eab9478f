"""GPU check of the device number conversions over all 2^32 fp32 bit
patterns (the formats the pages fix: first-level constants in an 8-bit
float, products in bf16; diycv.top "QLoRA 论文解读", section 关键公式, the
dtype table).

qlora_check_conversions applies the library's own device helpers (the
packed-pair fp32 -> bf16 rounding and the fp32 -> E4M3 encoder every kernel
uses) to consecutive bit patterns. Each chunk of 2^24 results is hashed and
compared with the SHA-256 that tests/golden/make_conversion_digests.py
stored from the oracle (oracle.nf4.bf16_rne, oracle.nf4.e4m3_encode) over
the same patterns; on a mismatch the oracle is run on that chunk to name
the first differing pattern. The E4M3 decoder is compared with
oracle.nf4.e4m3_decode on all 256 codes.
"""

import hashlib
import json
import os
import sys

import numpy as np
import pytest

from oracle import nf4
from gpu_util import require_gpu, say

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_conversion_digests as digests  # noqa: E402

pytestmark = pytest.mark.gpu
DIG = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "conversion_digests.json")))
CH = 1 << DIG["chunk_log2"]


@pytest.fixture(scope="module")
def api():
    return require_gpu()


def first_mismatch(chunk, got, kind):
    p = digests.patterns(chunk)
    x = p.view(np.float32)
    finite, bf16_ok = digests.domains(p)
    ok = bf16_ok if kind == "bf16" else finite
    ref = np.zeros(p.size, dtype=got.dtype)
    ref[ok] = nf4.bf16_rne(x[ok]) if kind == "bf16" else nf4.e4m3_encode(x[ok])
    bad = np.flatnonzero(ref != got)
    i = int(bad[0])
    return f"{kind}: {bad.size} patterns differ, first 0x{int(p[i]):08x}: device 0x{int(got[i]):x}, oracle 0x{int(ref[i]):x}"


@pytest.mark.parametrize("part", range(8))
def test_all_fp32_patterns(api, part):
    import torch

    nch = len(DIG["bf16_rne_uint16le"])
    per = nch // 8
    say(f"conversion sweep chunks {part * per} .. {part * per + per - 1} of {nch}")
    for chunk in range(part * per, part * per + per):
        bf, e8, _ = api.qlora_check_conversions(chunk * CH, CH)
        torch.cuda.synchronize()
        bfh = bf.cpu().numpy().view(np.uint16).copy()
        e8h = e8.cpu().numpy().copy()
        finite, bf16_ok = digests.domains(digests.patterns(chunk))
        bfh[~bf16_ok] = 0
        e8h[~finite] = 0
        if hashlib.sha256(bfh.tobytes()).hexdigest() != DIG["bf16_rne_uint16le"][chunk]:
            pytest.fail(first_mismatch(chunk, bfh, "bf16"))
        if hashlib.sha256(e8h.tobytes()).hexdigest() != DIG["e4m3_encode_uint8"][chunk]:
            pytest.fail(first_mismatch(chunk, e8h, "e4m3"))


def test_e4m3_decode_all_codes(api):
    import torch

    say("e4m3 decode table")
    _, _, tb = api.qlora_check_conversions(0, 0, bf16=False, e4m3=False, table=True)
    torch.cuda.synchronize()
    got = tb.cpu().numpy().astype(np.float64)
    ref = nf4.e4m3_decode(np.arange(256, dtype=np.uint8))
    live = ~np.isnan(ref)                      # codes 0x7F and 0xFF are NaN
    assert live.sum() == 254
    np.testing.assert_array_equal(got[live], ref[live])
