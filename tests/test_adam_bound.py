"""CPU checks of the Adam parity helpers (tests/adam_fp32.py).

The fp32 evaluation of clipped Adam steps must stay inside the error bound
derived from its roundings around the float64 oracle, element by element,
over several steps; and the bound must be tight enough to catch the
mistakes a kernel could plausibly make: the hyperparameter 0.999 taken in
float64 instead of the fp32 value the kernel receives (a 1.3e-5 relative
shift of 1 - beta2), a missing bias correction, or an unclipped gradient.
"""

import numpy as np
import pytest

from adam_fp32 import adam_error_bounds, adam_step_fp32
from oracle import optim

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8)


def run_fp32(theta0, grads, coefs, wd, step=adam_step_fp32):
    th = theta0.astype(np.float32)
    m = np.zeros_like(th)
    v = np.zeros_like(th)
    for t, (g, c) in enumerate(zip(grads, coefs), start=1):
        th, m, v = step(th, g, m, v, t, HP["lr"], HP["beta1"], HP["beta2"], HP["eps"], wd, c)
    return th, m, v


def inputs(n, seed):
    rng = np.random.default_rng(seed)
    theta0 = (0.02 * rng.standard_normal(n)).astype(np.float32)
    grads = [(s * rng.standard_normal(n)).astype(np.float32) for s in (0.001, 0.1, 0.5, 0.01, 2.0)]
    coefs = [np.float32(optim.clip_coef(g, 0.3)) for g in grads]
    return theta0, grads, coefs


@pytest.mark.parametrize("n,wd", [(20011, 0.0), (4099, 0.01)])
def test_fp32_evaluation_within_bound(n, wd):
    theta0, grads, coefs = inputs(n, n)
    th, m, v = run_fp32(theta0, grads, coefs, wd)
    rt, rm, rv, et, em, ev = adam_error_bounds(theta0, grads, [float(c) for c in coefs], wd=wd, **HP)
    assert np.all(np.abs(m - rm) <= em)
    assert np.all(np.abs(v - rv) <= ev)
    assert np.all(np.abs(th - rt) <= et)
    # the bound is a few fp32 roundings, not a blanket tolerance
    assert np.median(ev / rv) < 2e-6 and np.median(et / np.abs(rt)) < 1e-6


def test_bound_catches_plausible_mistakes():
    theta0, grads, coefs = inputs(5003, 1)
    rt, rm, rv, et, em, ev = adam_error_bounds(theta0, grads, [float(c) for c in coefs], wd=0.0, **HP)

    def beta2_in_float64(th, g, m, v, t, lr, b1, b2, eps, wd, c):
        # 1 - 0.999 formed from the decimal value instead of the fp32 beta2
        f = np.float32
        gc = f(c) * g
        m = f(b1) * m + f(1.0 - float(f(b1))) * gc
        v = f(b2) * v + f(1.0 - 0.999) * (gc * gc)
        upd = (m / f(1.0 - float(f(b1)) ** t)) / (np.sqrt(v / f(1.0 - float(f(b2)) ** t)) + f(eps))
        return th - f(lr) * upd, m, v

    def no_bias_correction(th, g, m, v, t, lr, b1, b2, eps, wd, c):
        f = np.float32
        gc = f(c) * g
        m = f(b1) * m + f(1.0 - float(f(b1))) * gc
        v = f(b2) * v + f(1.0 - float(f(b2))) * (gc * gc)
        return th - f(lr) * (m / (np.sqrt(v) + f(eps))), m, v

    _, _, v = run_fp32(theta0, grads, coefs, 0.0, beta2_in_float64)
    assert np.any(np.abs(v - rv) > ev)
    th, _, _ = run_fp32(theta0, grads, coefs, 0.0, no_bias_correction)
    assert np.any(np.abs(th - rt) > et)
    th, _, _ = run_fp32(theta0, grads, [np.float32(1.0)] * len(grads), 0.0)
    assert np.any(np.abs(th - rt) > et)
