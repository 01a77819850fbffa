"""fp64 chunkwise form of gated linear attention, with its intermediates.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: page "Gated Linear Attention Transformers with Hardware-Efficient Training"
(atlas.scime.ai summary), section Approach: an I/O-aware chunkwise algorithm with
inter-chunk states, a two-level (secondary) chunking of the intra-chunk part, and a
closed-form gate gradient; the chunkwise linear-attention form itself is credited on the
page "Transformer Quality in Linear Time" (science.uptrusthq.com, citation list) to
Hua et al. 2022.

Notation, per batch/head, with chunk size C, N = ceil(T/C) chunks, sub-chunk size c:
  g        chunk-local inclusive cumsum of log_alpha (restarts at every chunk)
  gamma_i  g at the last row of chunk i (the chunk's total log decay)
  S_[i]    state before chunk i (S_[0] = S0, S_[N] = S_T)
  Qh = Q * exp(g), Kh = K * exp(gamma - g)            (both factors <= 1)
  S_[i+1] = diag(exp(gamma_i)) S_[i] + Kh_i^T V_i
  O_i     = Qh_i S_[i] + A_i V_i,  A_ts = sum_d q_td k_sd exp(g_td - g_sd) for s <= t.
Two-level chunking of A (rows split into sub-chunks of c): a sub-block with t and s in
different sub-chunks I > J is formed as (Q_I * exp(g_I - g_rho)) (K_J * exp(g_rho - g_J))^T
with rho the first row of sub-chunk I, so both factors lie in [0,1]; a sub-block with t
and s in the same sub-chunk is formed element by element from log-space differences
exp(g_t - g_s).  In exact arithmetic the two give the same A; this module asserts the
exponent signs the rebasing relies on.

The backward mirrors it (derived by differentiating the chunk form; checked against the
step recurrence in the tests):
  dS_[N] = dS_T,  dS_[i] = diag(exp(gamma_i)) dS_[i+1] + Qh_i^T dO_i,  dS0 = dS_[0]
  dA  = tril(dO V^T)
  dQ  = (dO S_[i]^T) * exp(g)          + sum_{s<=t} dA_ts k_s * exp(g_t - g_s)
  dK  = (V dS_[i+1]^T) * exp(gamma - g) + sum_{t>=s} dA_ts q_t * exp(g_t - g_s)
  dV  = Kh dS_[i+1] + A^T dO
  dlog_alpha_t = sum_{u>=t} (q_u*dq_u - k_u*dk_u) + rowsum(dS_T * S_T)   (the closed form)
the last sum taken in two levels: a chunk-local suffix sum plus the suffix of chunk totals.
"""
from __future__ import annotations

import numpy as np

__all__ = ["gate_cumsum", "chunk_states", "intra_A", "chunkwise_fwd", "chunkwise_bwd"]

_F = np.float64


def _f64(x):
    return None if x is None else np.asarray(x, dtype=_F)


def _chunks(T, C):
    return [(s, min(T, s + C)) for s in range(0, T, C)]


def gate_cumsum(log_alpha, C):
    """Chunk-local inclusive cumsum g [..., T, dk] and chunk totals gamma [..., N, dk]."""
    la = _f64(log_alpha)
    T = la.shape[-2]
    g = np.empty_like(la)
    gam = []
    for s, e in _chunks(T, C):
        g[..., s:e, :] = np.cumsum(la[..., s:e, :], axis=-2)
        gam.append(g[..., e - 1, :])
    if not gam:
        return g, np.zeros(la.shape[:-2] + (0, la.shape[-1]), _F)
    return g, np.stack(gam, axis=-2)


def chunk_states(k, v, g, gamma, C, S0=None):
    """Inter-chunk recurrence.  Returns (states [..., N, dk, dv] = S_[0..N-1], S_T)."""
    k, v, g, gamma, S0 = map(_f64, (k, v, g, gamma, S0))
    lead, T, dk = k.shape[:-2], k.shape[-2], k.shape[-1]
    dv = v.shape[-1]
    S = np.zeros(lead + (dk, dv), _F) if S0 is None else S0.copy()
    states = []
    for i, (s, e) in enumerate(_chunks(T, C)):
        states.append(S.copy())
        gam = gamma[..., i, :]
        Kh = k[..., s:e, :] * np.exp(gam[..., None, :] - g[..., s:e, :])
        S = np.exp(gam)[..., :, None] * S + np.swapaxes(Kh, -1, -2) @ v[..., s:e, :]
    st = np.stack(states, axis=-3) if states else np.zeros(lead + (0, dk, dv), _F)
    return st, S


def _diag_block(q_rows, k_rows, g_q, g_k):
    """sum_d q_td k_sd exp(g_td - g_sd) for all (t, s) of one sub-chunk, s <= t."""
    n = q_rows.shape[-2]
    diff = g_q[..., :, None, :] - g_k[..., None, :, :]
    causal = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
    assert np.all(np.where(causal, diff, -1.0) <= 1e-12)
    dec = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    return np.sum(q_rows[..., :, None, :] * k_rows[..., None, :, :] * dec, axis=-1)


def intra_A(q, k, g, C, c):
    """Intra-chunk decayed attention matrices A [..., N, C, C] (zero above the diagonal
    and outside a ragged last chunk), built with two-level chunking."""
    q, k, g = map(_f64, (q, k, g))
    lead, T = q.shape[:-2], q.shape[-2]
    out = []
    for s0, e0 in _chunks(T, C):
        L = e0 - s0
        A = np.zeros(lead + (C, C), _F)
        Q, K, G = q[..., s0:e0, :], k[..., s0:e0, :], g[..., s0:e0, :]
        subs = _chunks(L, c)
        for I, (a, b) in enumerate(subs):
            rho = a
            qI = Q[..., a:b, :] * np.exp(G[..., a:b, :] - G[..., rho:rho + 1, :])
            for J, (a2, b2) in enumerate(subs[:I]):
                ex = G[..., rho:rho + 1, :] - G[..., a2:b2, :]
                assert np.all(ex <= 1e-12), "rebased exponent must be <= 0"
                kJ = K[..., a2:b2, :] * np.exp(ex)
                A[..., a:b, a2:b2] = qI @ np.swapaxes(kJ, -1, -2)
            A[..., a:b, a:b] = _diag_block(Q[..., a:b, :], K[..., a:b, :],
                                           G[..., a:b, :], G[..., a:b, :])
        out.append(A)
    if not out:
        return np.zeros(lead + (0, C, C), _F)
    return np.stack(out, axis=-3)


def chunkwise_fwd(q, k, v, log_alpha, S0=None, C=64, c=16):
    """Chunkwise forward.  Returns (o, S_T, intermediates dict)."""
    q, k, v, la, S0 = map(_f64, (q, k, v, log_alpha, S0))
    T = q.shape[-2]
    g, gamma = gate_cumsum(la, C)
    states, S_T = chunk_states(k, v, g, gamma, C, S0)
    A = intra_A(q, k, g, C, c)
    o = np.empty(v.shape[:-2] + (T, v.shape[-1]), _F)
    for i, (s, e) in enumerate(_chunks(T, C)):
        L = e - s
        Qh = q[..., s:e, :] * np.exp(g[..., s:e, :])
        o[..., s:e, :] = Qh @ states[..., i, :, :] + A[..., i, :L, :L] @ v[..., s:e, :]
    return o, S_T, dict(g=g, gamma=gamma, states=states, A=A)


def chunkwise_bwd(q, k, v, log_alpha, dO, S0=None, dS_T=None, C=64, c=16):
    """Chunkwise backward with the closed-form gate gradient.

    Returns (dq, dk, dv, dlog_alpha, dS0, intermediates dict).
    """
    q, k, v, la, dO, S0, dS_T = map(_f64, (q, k, v, log_alpha, dO, S0, dS_T))
    lead, T, dk_ = q.shape[:-2], q.shape[-2], q.shape[-1]
    dv_ = v.shape[-1]
    g, gamma = gate_cumsum(la, C)
    states, S_T = chunk_states(k, v, g, gamma, C, S0)
    A = intra_A(q, k, g, C, c)
    chunks = _chunks(T, C)
    N = len(chunks)

    # reverse inter-chunk recurrence of the state gradient; dstates[i] = dS_[i+1]
    dS = np.zeros(lead + (dk_, dv_), _F) if dS_T is None else dS_T.copy()
    dstates = [None] * N
    for i in reversed(range(N)):
        s, e = chunks[i]
        dstates[i] = dS.copy()
        Qh = q[..., s:e, :] * np.exp(g[..., s:e, :])
        dS = np.exp(gamma[..., i, :])[..., :, None] * dS + np.swapaxes(Qh, -1, -2) @ dO[..., s:e, :]
    dS0 = dS

    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for i, (s, e) in enumerate(chunks):
        L = e - s
        Q, K, V, G, dOc = q[..., s:e, :], k[..., s:e, :], v[..., s:e, :], g[..., s:e, :], dO[..., s:e, :]
        gam = gamma[..., i, None, :]
        Si, dSn = states[..., i, :, :], dstates[i]
        Ai = A[..., i, :L, :L]
        dA = np.tril(dOc @ np.swapaxes(V, -1, -2))
        # inter-chunk parts
        dQc = (dOc @ np.swapaxes(Si, -1, -2)) * np.exp(G)
        dKc = (V @ np.swapaxes(dSn, -1, -2)) * np.exp(gam - G)
        dVc = (K * np.exp(gam - G)) @ dSn + np.swapaxes(Ai, -1, -2) @ dOc
        # intra-chunk parts, two-level
        subs = _chunks(L, c)
        for I, (a, b) in enumerate(subs):
            rho = a
            eq = np.exp(G[..., a:b, :] - G[..., rho:rho + 1, :])       # <= 1
            qI = Q[..., a:b, :] * eq
            accq = np.zeros(lead + (b - a, dk_), _F)
            for J, (a2, b2) in enumerate(subs[:I]):
                ek = np.exp(G[..., rho:rho + 1, :] - G[..., a2:b2, :])  # <= 1
                assert np.all(ek <= 1.0 + 1e-12)
                dAIJ = dA[..., a:b, a2:b2]
                accq += dAIJ @ (K[..., a2:b2, :] * ek)
                dKc[..., a2:b2, :] += ek * (np.swapaxes(dAIJ, -1, -2) @ qI)
            dQc[..., a:b, :] += eq * accq
            # diagonal sub-block, log-space
            n = b - a
            diff = G[..., a:b, None, :] - G[..., None, a:b, :]          # [t, s, d]
            causal = np.tril(np.ones((n, n), dtype=bool))[:, :, None]
            dec = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
            dAd = dA[..., a:b, a:b][..., :, :, None]
            dQc[..., a:b, :] += np.sum(dAd * K[..., None, a:b, :] * dec, axis=-2)
            dKc[..., a:b, :] += np.sum(dAd * Q[..., a:b, None, :] * dec, axis=-3)
        dq[..., s:e, :] = dQc
        dk[..., s:e, :] = dKc
        dv[..., s:e, :] = dVc

    # closed-form gate gradient, two-level reverse cumsum
    Dt = q * dq - k * dk
    Dloc = np.empty_like(Dt)
    tot = []
    for s, e in chunks:
        Dloc[..., s:e, :] = np.flip(np.cumsum(np.flip(Dt[..., s:e, :], -2), -2), -2)
        tot.append(Dloc[..., s, :])
    dla = np.empty_like(Dt)
    carry = np.zeros(lead + (dk_,), _F)
    if dS_T is not None:
        carry = carry + np.sum(dS_T * S_T, axis=-1)
    for i in reversed(range(N)):
        s, e = chunks[i]
        dla[..., s:e, :] = Dloc[..., s:e, :] + carry[..., None, :]
        carry = carry + tot[i]
    inter = dict(g=g, gamma=gamma, states=states, S_T=S_T, A=A,
                 dstates=np.stack(dstates, axis=-3) if N else None, D_local=Dloc)
    return dq, dk, dv, dla, dS0, inter
