"""CPU checks of the seeded input generators (bit_nf4_quantized_amd/workloads.py).

The generators hold none of the method's arithmetic; these checks pin the
distributions they claim to draw. The Student-t draws (4 degrees of
freedom, the LLaMA-33B-shaped workload's heavy-tailed weights) are compared
with the closed-form CDF of t(4), F(t) = 1/2 + (3/4) x - x^3 / 4 with
x = t / sqrt(t^2 + 4), which follows from integrating the t(4) density
(3/8) (1 + t^2/4)^(-5/2).
"""

import numpy as np
import pytest

from bit_nf4_quantized_amd import workloads


def t4_cdf(t):
    x = t / np.sqrt(t * t + 4.0)
    return 0.5 + 0.75 * x - 0.25 * x ** 3


def test_t4_cdf_closed_form():
    # F(0) = 1/2, F(-t) = 1 - F(t), F'(0) = density at 0 = 3/8
    assert t4_cdf(0.0) == 0.5
    assert t4_cdf(-1.7) == pytest.approx(1.0 - t4_cdf(1.7), abs=1e-15)
    h = 1e-6
    assert (t4_cdf(h) - t4_cdf(-h)) / (2 * h) == pytest.approx(3.0 / 8.0, rel=1e-9)
    assert t4_cdf(1e6) == pytest.approx(1.0, abs=1e-12)


def test_student_t4_draws_match_the_t4_distribution():
    n = 2_000_000
    t = workloads.student_t4(np.random.default_rng(0), n)
    # Kolmogorov-Smirnov distance against the closed-form CDF: the 0.1 %
    # critical value for n = 2e6 is 1.95 / sqrt(n) ~ 1.4e-3
    ts = np.sort(t)
    F = t4_cdf(ts)
    i = np.arange(1, n + 1)
    d = max(np.max(i / n - F), np.max(F - (i - 1) / n))
    assert d < 1.95 / np.sqrt(n)
    # a normal of the same variance is far away (heavier tails)
    z = np.sort(np.sqrt(2.0) * np.random.default_rng(1).standard_normal(n))
    Fz = t4_cdf(z)
    assert max(np.max(i / n - Fz), np.max(Fz - (i - 1) / n)) > 10 / np.sqrt(n)


def test_student_t4_weight_std():
    w = workloads.draw_weight(np.random.default_rng(5), 1024, 1024, "student-t4", 0.02)
    assert w.dtype == np.float32 and w.shape == (1024, 1024)
    # t(4) has variance 2 but an infinite fourth moment: the sample std of a
    # million draws is within a few % of 0.02, and the tails are heavy
    assert abs(float(w.std()) - 0.02) < 0.002
    assert float(np.mean(np.abs(w) > 5 * 0.02)) > 10 * 5.7e-7
