"""Test helpers for the Adam step's parity (no GPU code).

* ``adam_step_fp32``: the textbook Adam update (Kingma and Ba, ICLR 2015,
  Algorithm 1; the pages' settings: diycv.top "QLoRA 论文解读", section
  训练与推理流程) evaluated in IEEE fp32 with one rounding per operation, in
  the order the update is written:
      gc = coef g
      m  = b1 m + (1 - b1) gc
      v  = b2 v + (1 - b2) (gc gc)
      upd = (m / bc1) / (sqrt(v / bc2) + eps)
      theta = theta - lr (upd + wd theta)
  with bc1 = fp32(1 - b1^t), bc2 = fp32(1 - b2^t) formed in float64 and
  rounded once, and 1 - b1, 1 - b2 exact (Sterbenz: b in [1/2, 1)).
  numpy float32 arithmetic is IEEE round-to-nearest-even with no fused
  multiply-add, and its sqrt and division are correctly rounded, so a
  kernel with the same operation order must match it bit for bit.

* ``adam_error_bounds``: per-element bounds on |fp32 result - exact result|
  after a run of clipped Adam steps, propagated step by step from the fp32
  roundings (unit roundoff u = 2^-24 per operation) along the float64
  trajectory. The fp32 coefficient may differ from the exact one by one
  rounding (plus 1e-15 relative for a float64 norm summed in another
  order). Second-order terms are covered by a 1 % margin and the float64
  trajectory's own rounding by 1e-14 relative.
"""

from __future__ import annotations

import numpy as np

U = 2.0 ** -24
TINY = 2.0 ** -149     # absolute error of one rounding into the subnormal range


def adam_step_fp32(theta, g, m, v, t: int, lr, beta1, beta2, eps, wd, coef):
    f = np.float32
    lr, b1, b2, eps, wd, c = f(lr), f(beta1), f(beta2), f(eps), f(wd), f(coef)
    omb1 = f(1.0 - float(b1))
    omb2 = f(1.0 - float(b2))
    bc1 = f(1.0 - float(b1) ** t)
    bc2 = f(1.0 - float(b2) ** t)
    theta, g, m, v = (np.asarray(a, dtype=np.float32) for a in (theta, g, m, v))
    gc = c * g
    m = b1 * m + omb1 * gc
    v = b2 * v + omb2 * (gc * gc)
    mh = m / bc1
    vh = v / bc2
    upd = mh / (np.sqrt(vh) + eps)
    theta = theta - lr * (upd + wd * theta)
    return theta.astype(np.float32), m.astype(np.float32), v.astype(np.float32)


def adam_error_bounds(theta0, grads, coefs, lr, beta1, beta2, eps, wd):
    """Run the float64 oracle (oracle.optim.adam_step) over ``grads`` with
    clip coefficients ``coefs`` and the fp32 hyperparameter values the
    kernel receives, and return (theta, m, v, e_theta, e_m, e_v): the
    oracle's results and per-element bounds on the error of an fp32
    evaluation of the same steps."""
    from oracle import optim

    th = np.asarray(theta0, dtype=np.float64)
    n = th.size
    m = np.zeros(n)
    v = np.zeros(n)
    em = np.zeros(n)
    ev = np.zeros(n)
    eth = np.zeros(n)
    b1, b2, lr, eps, wd = (float(np.float32(x)) for x in (beta1, beta2, lr, eps, wd))
    omb1, omb2 = 1.0 - b1, 1.0 - b2
    # relative error of the fp32 clipped gradient: the coefficient's fp32
    # rounding (+ a float64 norm summed in another order) and the product's
    gc_rel = 3.0 * U + 2e-15
    for t, (g, c) in enumerate(zip(grads, coefs), start=1):
        a = np.abs(float(c) * np.asarray(g, dtype=np.float64))
        th_new, m_new, v_new = optim.adam_step(th, g, m, v, t, lr, b1, b2, eps, wd, float(c))
        # m = RN(RN(b1 m) + RN(omb1 gc)): propagated error, the two products' and the sum's roundings
        em = (b1 * em * (1 + U) + U * b1 * np.abs(m) + omb1 * a * (gc_rel * (1 + U) + U)
              + U * (np.abs(m_new) + b1 * em + omb1 * a * gc_rel) + 3 * TINY) * 1.01
        # v = RN(RN(b2 v) + RN(omb2 RN(gc gc))): gc^2 carries twice gc's relative error
        ev = (b2 * ev * (1 + U) + U * b2 * v + omb2 * a * a * (2 * gc_rel + U) * (1 + U) + omb2 * a * a * U
              + U * (v_new + b2 * ev + 3 * omb2 * a * a * gc_rel) + 4 * TINY) * 1.01
        m, v = m_new, v_new
        bc1 = 1.0 - b1 ** t
        bc2 = 1.0 - b2 ** t
        mh = m / bc1
        vh = v / bc2
        # fp32 bc1, bc2 (one rounding each) and the division's rounding
        d_mh = em / bc1 + 2.001 * U * np.abs(mh) + TINY
        d_vh = ev / bc2 + 2.001 * U * vh + TINY
        sq = np.sqrt(vh)
        with np.errstate(divide="ignore", invalid="ignore"):
            lin = np.where(sq > 0, d_vh / (2 * sq), np.inf)
        d_sq = np.minimum(lin, np.sqrt(d_vh))          # |sqrt(a) - sqrt(b)| <= sqrt(|a - b|)
        d_sq = d_sq + U * (sq + d_sq)
        den = sq + eps
        d_den = d_sq + U * (den + d_sq)
        den_lo = np.maximum(den - d_den, eps * 0.5)
        upd = mh / den
        d_upd = d_mh / den_lo + np.abs(mh) * d_den / (den * den_lo)
        d_upd = d_upd + U * (np.abs(upd) + d_upd) + TINY
        w = wd * th
        d_w = wd * eth + U * abs(wd) * (np.abs(th) + eth) + (TINY if wd else 0.0)
        s = upd + w
        d_s = d_upd + d_w + U * (np.abs(s) + d_upd + d_w)
        p = lr * s
        d_p = lr * d_s + U * (np.abs(p) + lr * d_s) + TINY
        eth = (eth + d_p + U * (np.abs(th_new) + eth + d_p)) * 1.01
        th = th_new
    slack = 1e-14      # the float64 trajectory's own rounding
    return th, m, v, eth + slack * np.abs(th), em + slack * np.abs(m), ev + slack * v
