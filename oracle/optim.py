"""AdamW step for the adapter parameters -- plain CPU oracle in float64.

TEST INFRASTRUCTURE ONLY: imported by tests and the benchmark's CPU-baseline leg,
never by the product path.

[QLoRA-65B], the paged-optimizer entry of "메모리 회계": the adapters' Adam state
(m, v) lives in CPU pinned memory and is updated beside the backward. The update
rule is AdamW with decoupled weight decay (Loshchilov and Hutter, "Decoupled
Weight Decay Regularization", Algorithm 2 with a constant schedule multiplier),
which the pages do not spell out; the library applies the decay before the
moment update, as written here:

    p <- p (1 - lr wd)
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    p <- p - lr m_hat / (sqrt(v_hat) + eps),  m_hat = m / (1 - b1^t), v_hat = v / (1 - b2^t)

Hyperparameters are taken as the float32 values the library receives, then
everything is evaluated in float64.
"""

from __future__ import annotations

import numpy as np


def adamw_step(p, m, v, g, step: int, lr: float, beta1: float, beta2: float, eps: float, weight_decay: float):
    """Return (p, m, v) after step `step` (>= 1), all float64."""
    f = lambda a: float(np.float32(a))
    lr, b1, b2, eps, wd = f(lr), f(beta1), f(beta2), f(eps), f(weight_decay)
    p = np.asarray(p, dtype=np.float64) * (1.0 - lr * wd)
    g = np.asarray(g, dtype=np.float64)
    m = b1 * np.asarray(m, dtype=np.float64) + (1.0 - b1) * g
    v = b2 * np.asarray(v, dtype=np.float64) + (1.0 - b2) * g * g
    m_hat = m / (1.0 - b1 ** step)
    v_hat = v / (1.0 - b2 ** step)
    return p - lr * m_hat / (np.sqrt(v_hat) + eps), m, v
