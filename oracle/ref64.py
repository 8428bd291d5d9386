"""fp64 restatements used only to pin the fp32 oracle -- TEST INFRASTRUCTURE.

``adamw_fp64`` is the update of "Fused optimizers and state precision"
(ai-infra-kb M041), section 02, evaluated in float64 with numpy on whole
arrays; it serves as a higher-precision brute-force reference on tiny inputs,
where the fp32 oracle must agree to within fp32 rounding.  ``adam_l2_fp64`` is
the coupled-L2 route that the same section says is *not* AdamW (decay added to
the gradient before the moments); it exists for the negative test.
"""
from __future__ import annotations

import numpy as np


def adamw_fp64(theta, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """One step on float64 arrays; returns (theta, m, v, t)."""
    t = t + 1
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    theta = theta * (1.0 - lr * weight_decay) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return theta, m, v, t


def adam_l2_fp64(theta, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """Coupled L2: decay folded into the gradient (not AdamW)."""
    t = t + 1
    g = g + weight_decay * theta
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    theta = theta - lr * m_hat / (np.sqrt(v_hat) + eps)
    return theta, m, v, t
