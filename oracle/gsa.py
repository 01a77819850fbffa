"""Gated Slot Attention (GSA), fp64 (TEST INFRASTRUCTURE ONLY: see oracle/__init__.py).

Page "Gated Slot Attention for Efficient Linear-Time Sequence Modeling" (mlsanity.com
summary, Abstract): GSA keeps a bounded set of m memory slots (attention with
bounded-memory control) whose contents are forgotten adaptively by a GLA-style gate, and
reads them with a softmax; the layer is two GLA passes joined by a softmax.  Reading
taken (the page prints no formula): per batch and head, with a per-slot forget gate
alpha_t in (0, 1)^m and write strength 1 - alpha_t,

    Kt_t = diag(alpha_t) Kt_{t-1} + (1 - alpha_t)^T k_t      (m x dk key slots)
    Vt_t = diag(alpha_t) Vt_{t-1} + (1 - alpha_t)^T v_t      (m x dv value slots)
    o_t  = softmax(Kt_t q_t)^T Vt_t                           (softmax over the m slots)

from zero slots.  The first pass, s_t = Kt_t q_t, is a GLA whose gate acts on the output
(slot) dimension; the second, o_t = p_t Vt_t with p_t = softmax(s_t), is the key-gated GLA
of the main layer with queries p, keys 1 - alpha and values v.

`gsa_fwd` is the step recurrence above; `gsa_bwd` differentiates that same recurrence
with torch autograd in float64 on the CPU (a library primitive for the chain rule of the
written forward).  `two_pass_fwd` evaluates the two-GLA form (an explicit value-gated sum,
a softmax, the main layer's recurrence) and is one of the pins.
"""
from __future__ import annotations

import numpy as np

from .recurrence import recurrence_fwd


def _steps_torch(q, k, v, la):
    import torch
    T = q.shape[0]
    m = la.shape[1]
    Kt = torch.zeros((m, q.shape[1]), dtype=torch.float64)
    Vt = torch.zeros((m, v.shape[1]), dtype=torch.float64)
    outs = []
    for t in range(T):
        a = torch.exp(la[t])
        Kt = a[:, None] * Kt + (1.0 - a)[:, None] * k[t][None, :]
        Vt = a[:, None] * Vt + (1.0 - a)[:, None] * v[t][None, :]
        p = torch.softmax(Kt @ q[t], dim=0)
        outs.append(p @ Vt)
    return torch.stack(outs)


def gsa_fwd(q, k, v, log_alpha):
    """o [T, dv] for one batch/head: q, k [T, dk], v [T, dv], log_alpha [T, m] (<= 0)."""
    import torch
    args = [torch.as_tensor(np.asarray(x, dtype=np.float64)) for x in (q, k, v, log_alpha)]
    with torch.no_grad():
        return _steps_torch(*args).numpy()


def gsa_bwd(q, k, v, log_alpha, dO):
    """dq, dk, dv, dlog_alpha for the loss sum(o * dO)."""
    import torch
    args = [torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True)
            for x in (q, k, v, log_alpha)]
    o = _steps_torch(*args)
    grads = torch.autograd.grad(o, args, grad_outputs=torch.as_tensor(np.asarray(dO, dtype=np.float64)))
    return tuple(g.numpy() for g in grads)


def value_gated_scores(q, k, w, log_alpha):
    """The first pass written as a sum: s_t[j] = sum_{u<=t} (q_t . k_u) w_u[j]
    exp(L_t[j] - L_u[j]), L the inclusive cumulative sum of log_alpha over time."""
    q, k, w, la = (np.asarray(x, dtype=np.float64) for x in (q, k, w, log_alpha))
    L = np.cumsum(la, axis=0)
    T = q.shape[0]
    s = np.zeros((T, w.shape[1]))
    for t in range(T):
        for u in range(t + 1):
            s[t] += (q[t] @ k[u]) * w[u] * np.exp(L[t] - L[u])
    return s


def two_pass_fwd(q, k, v, log_alpha):
    """GSA as two GLA passes joined by a softmax (for small T)."""
    la = np.asarray(log_alpha, dtype=np.float64)
    w = 1.0 - np.exp(la)
    s = value_gated_scores(q, k, w, la)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o, _ = recurrence_fwd(p, w, v, la)
    return o
