"""Pins of the oracle's scalar-gate variants (oracle/scalar.py) against facts that do not
come from it: the state written out as an explicit sum of decayed outer products, the
RetNet-style decay matrix gamma^(t-s) by integer powers, plain causal linear attention
when the gate is 1, and the gradient with respect to the scalar gates by finite
differences of the forward."""
import numpy as np

from oracle import scalar


def _inputs(seed, T=12, dk=3, dv=4):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    v, dO = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    la = -np.abs(rng.standard_normal(T)) * 0.3
    S0, dST = rng.standard_normal((dk, dv)), rng.standard_normal((dk, dv))
    return q, k, v, dO, la, S0, dST


def test_state_and_output_as_explicit_decayed_sums():
    q, k, v, _, la, S0, _ = _inputs(1)
    T = q.shape[0]
    o, ST = scalar.scalar_fwd(q, k, v, la, S0)
    alpha = np.exp(la)
    for t in (0, 5, T - 1):
        # S_t = (prod_{u<=t} alpha_u) S0 + sum_{s<=t} (prod_{s<u<=t} alpha_u) k_s^T v_s
        S = np.prod(alpha[: t + 1]) * S0
        for s_ in range(t + 1):
            S = S + np.prod(alpha[s_ + 1: t + 1]) * np.outer(k[s_], v[s_])
        assert np.allclose(o[t], q[t] @ S, rtol=1e-12, atol=1e-12)
        if t == T - 1:
            assert np.allclose(ST, S, rtol=1e-12, atol=1e-12)


def test_matches_parallel_decay_matrix_form():
    q, k, v, _, la, S0, _ = _inputs(2, T=20)
    o, _ = scalar.scalar_fwd(q, k, v, la, S0)
    assert np.allclose(o, scalar.parallel_fwd(q, k, v, la, S0), rtol=1e-12, atol=1e-12)


def test_constant_decay_is_retnet_power_matrix():
    q, k, v, _, _, _, _ = _inputs(3, T=16)
    gamma = 1.0 - 2.0 ** -5          # a RetNet-style per-head decay
    la = np.full(16, np.log(gamma))
    t, s = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    D = np.where(t >= s, gamma ** np.maximum(t - s, 0).astype(np.float64), 0.0)
    assert np.allclose(scalar.decay_matrix(la), D, rtol=1e-13, atol=0)
    o, _ = scalar.scalar_fwd(q, k, v, la)
    assert np.allclose(o, ((q @ k.T) * D) @ v, rtol=1e-12, atol=1e-12)


def test_unit_gate_is_causal_linear_attention():
    q, k, v, _, _, _, _ = _inputs(4)
    o, ST = scalar.scalar_fwd(q, k, v, np.zeros(q.shape[0]))
    assert np.allclose(o, np.tril(q @ k.T) @ v, rtol=1e-12, atol=1e-12)
    assert np.allclose(ST, k.T @ v, rtol=1e-12, atol=1e-12)


def test_gradients_by_finite_differences():
    q, k, v, dO, la, S0, dST = _inputs(5, T=9)

    def loss(qq=q, kk=k, vv=v, ll=la, s0=S0):
        o, ST = scalar.scalar_fwd(qq, kk, vv, ll, s0)
        return float(np.sum(o * dO) + np.sum(ST * dST))

    dq, dk, dv, dla, dS0 = scalar.scalar_bwd(q, k, v, la, dO, S0, dST)
    assert dla.shape == la.shape
    h = 1e-6
    for t in range(la.shape[0]):
        lp, lm = la.copy(), la.copy()
        lp[t] += h
        lm[t] -= h
        fd = (loss(ll=lp) - loss(ll=lm)) / (2 * h)
        assert abs(fd - dla[t]) <= 1e-6 * max(1.0, abs(fd)), (t, fd, dla[t])
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv), ("S0", S0, dS0)):
        for idx in [(0, 0), (min(3, x.shape[0] - 1), 1), (x.shape[0] - 1, x.shape[1] - 1)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            kw = {"q": "qq", "k": "kk", "v": "vv", "S0": "s0"}[name]
            fd = (loss(**{kw: xp}) - loss(**{kw: xm})) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, idx, fd, g[idx])
