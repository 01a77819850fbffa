"""Step-by-step fp64 definition of gated linear attention and its exact gradients.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: page "Gated Linear Attention Transformers with Hardware-Efficient Training"
(atlas.scime.ai summary), section Approach: a linear-attention state with the
data-dependent low-rank gate G_t = alpha_t^T 1.  Applying G_t elementwise to the
dk x dv state scales row d by alpha_t[d], so the step is

    S_t = diag(alpha_t) S_{t-1} + outer(k_t, v_t),    o_t = q_t S_t,    S_{-1} = S0,

with alpha_t = exp(log_alpha_t).  The gate acts on the past only; the current token
enters with weight one and o_t reads the updated state (reading S1 in the design notes).
There is no normaliser, scale or output gate inside the layer (reading S2).

All arrays are float64 with layout [..., T, d] (any leading batch/head dims); states
are [..., dk, dv].
"""
from __future__ import annotations

import numpy as np

__all__ = ["recurrence_fwd", "recurrence_bwd", "quadratic_fwd", "closed_form_gate_grad"]

_F = np.float64


def _f64(x):
    return None if x is None else np.asarray(x, dtype=_F)


def recurrence_fwd(q, k, v, log_alpha, S0=None):
    """Forward recurrence, one token at a time.

    Returns (o [..., T, dv], S_T [..., dk, dv]).
    """
    q, k, v, la, S0 = map(_f64, (q, k, v, log_alpha, S0))
    lead, T, dk = q.shape[:-2], q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (dk, dv), _F) if S0 is None else S0.copy()
    o = np.empty(lead + (T, dv), _F)
    alpha = np.exp(la)
    for t in range(T):
        S *= alpha[..., t, :, None]                        # diag(alpha_t) S_{t-1}
        S += k[..., t, :, None] * v[..., t, None, :]       # + k_t^T v_t
        o[..., t, :] = (q[..., t, None, :] @ S)[..., 0, :]  # o_t = q_t S_t
    return o, S


def recurrence_bwd(q, k, v, log_alpha, dO, S0=None, dS_T=None, seg_budget_bytes=256 << 20):
    """Reverse-mode gradient of the loss  <o, dO> + <S_T, dS_T>  by direct
    differentiation of every step of `recurrence_fwd` (not the closed form).

    Per-step states are recomputed from fp64 checkpoints, one segment at a time.
    Returns (dq, dk, dv, dlog_alpha, dS0).
    """
    q, k, v, la, dO, S0, dS_T = map(_f64, (q, k, v, log_alpha, dO, S0, dS_T))
    lead, T, dk = q.shape[:-2], q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    state_bytes = int(np.prod(lead, dtype=np.int64)) * dk * dv * 8
    seg = int(max(1, min(64, seg_budget_bytes // max(state_bytes, 1))))
    alpha = np.exp(la)

    # forward sweep keeping S_{t0-1} at every segment start t0
    S = np.zeros(lead + (dk, dv), _F) if S0 is None else S0.copy()
    starts = list(range(0, T, seg))
    ckpt = {}
    for t in range(T):
        if t % seg == 0:
            ckpt[t] = S.copy()
        S *= alpha[..., t, :, None]
        S += k[..., t, :, None] * v[..., t, None, :]

    dq = np.empty_like(q)
    dk_ = np.empty_like(k)
    dv_ = np.empty_like(v)
    dla = np.empty_like(la)
    dS = np.zeros(lead + (dk, dv), _F) if dS_T is None else dS_T.copy()   # d loss / d S_{T-1}
    for t0 in reversed(starts):
        t1 = min(T, t0 + seg)
        # states[j] = S_{t0-1+j}, j = 0 .. t1-t0
        states = [ckpt[t0]]
        for t in range(t0, t1):
            Sn = states[-1] * alpha[..., t, :, None] + k[..., t, :, None] * v[..., t, None, :]
            states.append(Sn)
        for t in range(t1 - 1, t0 - 1, -1):
            S_t = states[t - t0 + 1]
            S_prev = states[t - t0]
            dS += q[..., t, :, None] * dO[..., t, None, :]          # o_t = q_t S_t
            dq[..., t, :] = (S_t @ dO[..., t, :, None])[..., 0]
            dk_[..., t, :] = (dS @ v[..., t, :, None])[..., 0]       # S_t += k_t^T v_t
            dv_[..., t, :] = (k[..., t, None, :] @ dS)[..., 0, :]
            # S_t = diag(alpha_t) S_{t-1}: d alpha_t[d] = sum_v dS[d,v] S_{t-1}[d,v]
            dla[..., t, :] = alpha[..., t, :] * np.sum(dS * S_prev, axis=-1)
            dS *= alpha[..., t, :, None]
    return dq, dk_, dv_, dla, dS


def quadratic_fwd(q, k, v, log_alpha, S0=None):
    """Parallel (attention-like) form for tiny T:

        o_t = sum_{s<=t} sum_d q_td k_sd exp(L_td - L_sd) v_s + (q_t * exp(L_t)) S0,

    with L the inclusive cumulative sum of log_alpha over the whole sequence.
    Memory is O(T^2 dk): use only for T of a few hundred at most.
    """
    q, k, v, la, S0 = map(_f64, (q, k, v, log_alpha, S0))
    T = q.shape[-2]
    L = np.cumsum(la, axis=-2)
    diff = L[..., :, None, :] - L[..., None, :, :]               # [..., t, s, d]
    causal = np.tril(np.ones((T, T), dtype=bool))
    decay = np.where(causal[:, :, None], np.exp(np.where(causal[:, :, None], diff, 0.0)), 0.0)
    W = np.sum(q[..., :, None, :] * k[..., None, :, :] * decay, axis=-1)   # [..., t, s]
    o = W @ v
    if S0 is not None:
        o = o + (q * np.exp(L)) @ S0
    return o


def closed_form_gate_grad(q, dq, k, dk, S_T=None, dS_T=None):
    """The pages' closed-form gate gradient (Approach section: a gate gradient that needs
    no per-step states): the reverse cumulative sum over time of q*dq - k*dk, plus, when
    a gradient dS_T flows into the final state, rowsum(dS_T * S_T) at every position.
    """
    q, dq, k, dk = map(_f64, (q, dq, k, dk))
    Dt = q * dq - k * dk
    out = np.flip(np.cumsum(np.flip(Dt, axis=-2), axis=-2), axis=-2)
    if dS_T is not None:
        out = out + np.sum(_f64(dS_T) * _f64(S_T), axis=-1)[..., None, :]
    return out
