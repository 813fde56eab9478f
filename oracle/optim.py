"""The adapters' optimiser step (CPU oracle). Test infrastructure only.

The pages' Guanaco runs train the LoRA adapters with Adam, beta2 = 0.999,
max grad norm 0.3 and a constant learning rate (page diycv.top "QLoRA
论文解读", section 训练与推理流程, common settings), with the optimiser
state paged between GPU and CPU memory (section 方法总览 item 4). Paging
moves the state, not the arithmetic, so the oracle is the plain step:

* global gradient-norm clipping over all adapter gradients: with
  n = sqrt(sum g^2), every gradient is multiplied by
  coef = min(1, max_norm / (n + 1e-6));
* Adam (Kingma and Ba, "Adam: A Method for Stochastic Optimization", ICLR
  2015, Algorithm 1), step t >= 1 on the clipped gradient g:
      m = beta1 m + (1 - beta1) g,    v = beta2 v + (1 - beta2) g^2,
      m_hat = m / (1 - beta1^t),      v_hat = v / (1 - beta2^t),
      theta = theta - lr (m_hat / (sqrt(v_hat) + eps) + wd theta)
  (wd, a decoupled weight decay, is 0 unless given).

Readings (also in the design notes): the parameters are kept in fp32 (the
layer reads their bf16 rounding), beta1 = 0.9 and eps = 1e-8 where the
pages give no value, and the 1e-6 in the clipping denominator and the
clamp at 1 follow the usual definition of clipping by total norm.
Everything here is float64.
"""

from __future__ import annotations

import numpy as np

_F64 = np.float64


def grad_norm(g) -> float:
    g = np.asarray(g, dtype=_F64).reshape(-1)
    return float(np.sqrt(np.sum(g * g)))


def clip_coef(g, max_norm: float) -> float:
    n = grad_norm(g)
    return float(min(1.0, float(max_norm) / (n + 1e-6)))


def adam_step(theta, g, m, v, t: int, lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8,
              wd: float = 0.0, coef: float = 1.0):
    """One Adam step on clipped gradient coef * g; returns (theta, m, v) as float64."""
    if t < 1:
        raise ValueError("step t starts at 1")
    theta, g, m, v = (np.asarray(a, dtype=_F64) for a in (theta, g, m, v))
    g = coef * g
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    theta = theta - lr * (m_hat / (np.sqrt(v_hat) + eps) + wd * theta)
    return theta, m, v
