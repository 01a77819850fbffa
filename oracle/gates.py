"""Gate front-end of the layer, fp64 (TEST INFRASTRUCTURE ONLY: see oracle/__init__.py).

Page "Gated Linear Attention Transformers with Hardware-Efficient Training" (atlas.scime.ai
summary, section Approach): the gate alpha_t is data-dependent.  The front-end offered by
the library takes per-(t, d) gate logits x and forms

    log_alpha = logsigmoid(x) / tau,      i.e. alpha = sigmoid(x) ** (1 / tau),

a gate in (0, 1) whose temperature tau > 0 keeps it near 1 (slow forgetting).  The
gradient of the layer with respect to x follows by the chain rule from the gradient with
respect to log_alpha:

    d logsigmoid(x) / dx = 1 - sigmoid(x) = sigmoid(-x),
    dL/dx = dL/dlog_alpha * sigmoid(-x) / tau.
"""
from __future__ import annotations

import numpy as np

from .recurrence import recurrence_bwd, recurrence_fwd


def logsigmoid(x):
    """log(sigmoid(x)) = min(x, 0) - log(1 + exp(-|x|)), finite for every finite x."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def sigmoid_neg(x):
    """sigmoid(-x) = 1 / (1 + exp(x)), computed without overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, e / (1.0 + e), 1.0 / (1.0 + e))


def log_alpha_from_logits(x, tau):
    return logsigmoid(x) / float(tau)


def logits_grad(dlog_alpha, x, tau):
    return np.asarray(dlog_alpha, dtype=np.float64) * sigmoid_neg(x) / float(tau)


def fwd_logits(q, k, v, x, tau, S0=None):
    """o, S_T of the layer fed gate logits x (one batch/head, [T, d])."""
    return recurrence_fwd(q, k, v, log_alpha_from_logits(x, tau), S0)


def bwd_logits(q, k, v, x, tau, dO, S0=None, dS_T=None):
    """dq, dk, dv, dx, dS0 of the layer fed gate logits x (one batch/head)."""
    la = log_alpha_from_logits(x, tau)
    dq, dk, dv, dla, dS0 = recurrence_bwd(q, k, v, la, dO, S0, dS_T)
    return dq, dk, dv, logits_grad(dla, x, tau), dS0
