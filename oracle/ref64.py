"""fp64 references used only to pin the fp32 oracle -- TEST INFRASTRUCTURE.

``adamw_fp64`` is the decoupled-decay AdamW step of "Fused optimizers and
state precision" (ai-infra-kb M041), section 02, carried out in float64 on
whole numpy arrays: the two moment averages, the bias corrections 1 - beta^t
taken as two scalars, and the step of theta made of a shrink by
(1 - lr * weight_decay) and an Adam direction of size lr.  It is a
higher-precision brute force for tiny inputs, where the fp32 oracle must agree
to within fp32 rounding.  ``adam_l2_fp64`` is the coupled-L2 route that the
same section sets apart from AdamW (the decay term joins the gradient before
the moments are formed, and theta is not shrunk); it exists for the negative
test.
"""
from __future__ import annotations

import numpy as np


def _adam_direction(m1, m2, count, b1, b2, eps):
    """Bias-corrected first moment over (root of the corrected second + eps)."""
    corr1 = 1.0 - np.power(b1, count)
    corr2 = 1.0 - np.power(b2, count)
    return (m1 / corr1) / (np.sqrt(m2 / corr2) + eps)


def adamw_fp64(theta, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """One step on float64 arrays; returns (theta, m, v, t)."""
    count = t + 1
    m_next = m + (1.0 - beta1) * (g - m)           # beta1*m + (1-beta1)*g
    v_next = v + (1.0 - beta2) * (g * g - v)       # beta2*v + (1-beta2)*g^2
    shrink = 1.0 - lr * weight_decay
    theta_next = shrink * theta - lr * _adam_direction(m_next, v_next, count, beta1, beta2, eps)
    return theta_next, m_next, v_next, count


def adam_l2_fp64(theta, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """Coupled L2: decay folded into the gradient (not AdamW)."""
    count = t + 1
    g_l2 = g + weight_decay * theta
    m_next = m + (1.0 - beta1) * (g_l2 - m)
    v_next = v + (1.0 - beta2) * (g_l2 * g_l2 - v)
    theta_next = theta - lr * _adam_direction(m_next, v_next, count, beta1, beta2, eps)
    return theta_next, m_next, v_next, count
