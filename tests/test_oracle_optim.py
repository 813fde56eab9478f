"""Pins of the optimiser oracle (oracle/optim.py): PyTorch's CPU Adam and
clip_grad_norm_ in float64 (independent implementations of the same
textbook definitions), and closed forms: the first step and a constant
gradient give updates of size lr (bias correction exact), a 3-4-5 gradient
has norm 5, gradient scaling leaves Adam's step unchanged, and decoupled
weight decay shrinks the parameters by lr wd theta.
"""

import numpy as np
import pytest

from oracle import optim


def test_matches_torch_adam_and_clipping_over_steps():
    import torch

    rng = np.random.default_rng(0)
    n = 1000
    theta0 = rng.standard_normal(n) * 0.02
    grads = [rng.standard_normal(n) * (0.05 + 0.5 * k) for k in range(6)]
    lr, b1, b2, eps, wd, max_norm = 2e-4, 0.9, 0.999, 1e-8, 0.01, 0.3
    p = torch.nn.Parameter(torch.tensor(theta0, dtype=torch.float64))
    opt = torch.optim.AdamW([p], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    theta, m, v = theta0.copy(), np.zeros(n), np.zeros(n)
    for t, g in enumerate(grads, start=1):
        p.grad = torch.tensor(g, dtype=torch.float64)
        torch.nn.utils.clip_grad_norm_([p], max_norm)
        opt.step()
        coef = optim.clip_coef(g, max_norm)
        # torch's AdamW decays before the Adam update: theta (1 - lr wd) - lr m_hat/(sqrt v_hat + eps),
        # which is the same expression as theta - lr (m_hat/(...) + wd theta)
        theta, m, v = optim.adam_step(theta, g, m, v, t, lr, b1, b2, eps, wd, coef)
        np.testing.assert_allclose(theta, p.detach().numpy(), rtol=0, atol=1e-15)
    st = opt.state[p]
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=0)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=0)


def test_clip_coefficient():
    assert optim.grad_norm([3.0, 4.0]) == 5.0
    assert optim.clip_coef([3.0, 4.0], 0.3) == pytest.approx(0.3 / (5.0 + 1e-6), rel=1e-15)
    assert optim.clip_coef([0.1, 0.1], 0.3) == 1.0          # below the limit: unchanged
    assert optim.clip_coef(np.zeros(10), 0.3) == 1.0


def test_first_step_and_constant_gradient_move_by_lr():
    g = np.array([0.5, -2.0, 1e-3, -7.0])
    theta = np.zeros(4)
    m = v = np.zeros(4)
    lr = 1e-3
    for t in range(1, 6):
        theta, m, v = optim.adam_step(theta, g, m, v, t, lr, eps=0.0)
        # bias correction makes m_hat = g and v_hat = g^2 for a constant gradient
        np.testing.assert_allclose(theta, -t * lr * np.sign(g), rtol=1e-12, atol=0)


def test_gradient_scale_invariance_and_weight_decay():
    rng = np.random.default_rng(1)
    g = rng.standard_normal(50)
    th = rng.standard_normal(50)
    a, _, _ = optim.adam_step(th, g, np.zeros(50), np.zeros(50), 1, 1e-2, eps=0.0)
    b, _, _ = optim.adam_step(th, 1000.0 * g, np.zeros(50), np.zeros(50), 1, 1e-2, eps=0.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    c, _, _ = optim.adam_step(th, np.zeros(50), np.zeros(50), np.zeros(50), 1, 1e-2, eps=1e-8, wd=0.5)
    np.testing.assert_allclose(c, th * (1 - 1e-2 * 0.5), rtol=1e-14)


def test_step_zero_is_rejected():
    with pytest.raises(ValueError):
        optim.adam_step([0.0], [1.0], [0.0], [0.0], 0, 1e-3)
