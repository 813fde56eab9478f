"""Pins for the oracle's NF4 codebook (CPU only).

The pages print no codebook values, so parity with any other NF4 table is
unpinned. The codebook is pinned instead by what the pages fix (16 values,
range [-1, 1], one exact zero, asymmetric; page diycv.top, section 方法总览
item 2; neura.market, "How It Works") and by properties of the quantile
construction checked through a different function than the one the oracle
uses (the normal CDF via erfc instead of the inverse CDF).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nf4_facts.json")


def phi(x: float) -> float:
    """Standard normal CDF through erfc (not the oracle's quantile routine)."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def quantile_by_bisection(p: float) -> float:
    """Independent N(0,1) quantile: bisection on the erfc-based CDF."""
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if phi(mid) < p:
            lo = mid
        else:
            hi = mid
        if hi - lo <= 0.0:
            break
    return 0.5 * (lo + hi)


@pytest.fixture(scope="module")
def facts():
    with open(GOLDEN) as f:
        return json.load(f)


def test_pages_invariants(facts):
    q = nf4.nf4_codebook()
    assert q.dtype == np.float32
    assert q.size == facts["n_codes"] == 2 ** facts["k"]
    assert np.all(np.diff(q.astype(np.float64)) > 0)           # strictly increasing
    assert q[0] == np.float32(facts["min"]) and q[-1] == np.float32(facts["max"])
    zeros = np.flatnonzero(q == 0)
    assert zeros.tolist() == [7]                               # exactly one zero
    assert not np.signbit(q[7])
    # asymmetric: 7 negative and 8 positive codes, and not mirror images
    assert int(np.sum(q < 0)) == 7 and int(np.sum(q > 0)) == 8
    assert not np.allclose(np.sort(-q), q)


def test_independent_quantile_gives_same_bits():
    a = nf4.nf4_codebook()
    b = nf4.nf4_codebook(quantile=quantile_by_bisection)
    assert a.view(np.uint32).tolist() == b.view(np.uint32).tolist()


@pytest.mark.parametrize("c", [15, 17])
def test_quantile_sets_lie_in_their_bins(c, facts):
    """Each q_i is the midpoint of the N(0,1) quantiles at i/d and (i+1)/d, so
    its CDF value lies strictly inside that probability bin. d = 2^k + 1 = 17
    for the pages' 15-value set; the 17-value set uses d = 19."""
    d = c + 2
    if c == 15:
        assert d == facts["quantile_denominator"]
    vals = nf4.quantile_midpoint_set(c)
    assert len(vals) == c
    for i, v in enumerate(vals, start=1):
        assert math.isfinite(v)
        p = phi(v)
        assert i / d < p < (i + 1) / d, (c, i, v, p)
    # symmetric with an exact middle zero
    assert vals[c // 2] == 0.0
    for i in range(c):
        assert vals[i] == pytest.approx(-vals[c - 1 - i], abs=1e-14)


def test_normalisation_of_the_two_halves():
    """Negative codes are the negative members of S_15 over |min S_15|,
    positive codes the positive members of S_17 over max S_17."""
    q = nf4.nf4_codebook().astype(np.float64)
    s15 = np.array(nf4.quantile_midpoint_set(15))
    s17 = np.array(nf4.quantile_midpoint_set(17))
    neg = s15[s15 < 0] / -s15.min()
    pos = s17[s17 > 0] / s17.max()
    np.testing.assert_allclose(q[:7], np.sort(neg), rtol=0, atol=2 ** -24)
    np.testing.assert_allclose(q[8:], np.sort(pos), rtol=0, atol=2 ** -24)


def test_midpoints_exact_and_ordered():
    q = nf4.nf4_codebook()
    m = nf4.nf4_midpoints(q)
    assert m.size == 15
    q64 = q.astype(np.float64)
    for j in range(15):
        assert q64[j] < m[j] < q64[j + 1]
        # exactness: 2*m_j - q_j recovers q_{j+1} exactly
        assert 2.0 * m[j] - q64[j] == q64[j + 1]
    # the largest half-gap bounds the normalised rounding error
    assert float(np.max(np.diff(q64)) / 2) < 0.116
