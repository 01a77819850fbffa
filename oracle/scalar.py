"""Scalar-gate variants of the layer, fp64 (TEST INFRASTRUCTURE ONLY: see
oracle/__init__.py).

Page "Gated Linear Attention Transformers with Hardware-Efficient Training" (atlas.scime.ai
summary, section Experiments, the ablation table and its take-aways): besides the
fine-grained gate (one decay per key dimension) the pages compare a data-dependent scalar
gate (one decay per token and head) and a data-independent scalar decay per head
(RetNet-style).  With a scalar gate alpha_t every row of the state decays alike:

    S_t = alpha_t S_{t-1} + k_t^T v_t,     o_t = q_t S_t,

which is the fine-grained layer with log_alpha_t repeated over the key dimension.  The
loss gradient with respect to the scalar log-gate is therefore the sum over the key
dimension of the fine-grained one.  A data-independent decay gamma_h is the case of a
log-gate constant along t (log gamma_h at every token).

The parallel form used by the pins: with D_ts = exp(sum of log_alpha_u for s < u <= t)
for s <= t and 0 above the diagonal,

    o = ((Q K^T) * D) V  (+ (q_t exp(L_t)) S0, L the inclusive cumulative sum).
"""
from __future__ import annotations

import numpy as np

from .recurrence import recurrence_bwd, recurrence_fwd


def broadcast(la_s, dk):
    """[..., T] scalar log-gates -> [..., T, dk] (the same value for every key dimension)."""
    la_s = np.asarray(la_s, dtype=np.float64)
    return np.repeat(la_s[..., None], dk, axis=-1)


def scalar_fwd(q, k, v, la_s, S0=None):
    """o, S_T of the layer with one gate per token (la_s [..., T])."""
    return recurrence_fwd(q, k, v, broadcast(la_s, np.shape(q)[-1]), S0)


def scalar_bwd(q, k, v, la_s, dO, S0=None, dS_T=None):
    """dq, dk, dv, dla_s, dS0 with dla_s [..., T] = the per-key gate gradient summed over
    the key dimension."""
    dq, dk, dv, dla, dS0 = recurrence_bwd(q, k, v, broadcast(la_s, np.shape(q)[-1]), dO, S0,
                                          dS_T)
    return dq, dk, dv, np.sum(dla, axis=-1), dS0


def decay_matrix(la_s):
    """D_ts = exp(sum_{s<u<=t} la_s[u]) for s <= t, else 0 ([..., T, T])."""
    la_s = np.asarray(la_s, dtype=np.float64)
    T = la_s.shape[-1]
    L = np.cumsum(la_s, axis=-1)
    diff = L[..., :, None] - L[..., None, :]
    causal = np.tril(np.ones((T, T), dtype=bool))
    return np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)


def parallel_fwd(q, k, v, la_s, S0=None):
    """The parallel form ((Q K^T) * D) V of the scalar-gated layer, for small T."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    o = ((q @ np.swapaxes(k, -1, -2)) * decay_matrix(la_s)) @ v
    if S0 is not None:
        L = np.cumsum(np.asarray(la_s, dtype=np.float64), axis=-1)
        o = o + (q * np.exp(L)[..., None]) @ np.asarray(S0, dtype=np.float64)
    return o
