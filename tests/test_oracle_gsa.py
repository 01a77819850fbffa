"""Pins of the oracle's Gated Slot Attention (oracle/gsa.py) against facts that do not
come from its step recurrence: the two-GLA-pass form (an explicit value-gated sum, a
softmax and the main layer's pinned recurrence), closed forms for one slot (the softmax
is 1: a gated running average of v) and for zero queries (uniform read of the value
slots), and every gradient by central finite differences of the forward."""
import numpy as np

from oracle import gsa


def _inputs(seed, T=8, dk=3, dv=4, m=5):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    v, dO = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    la = -np.abs(rng.standard_normal((T, m))) * 0.6
    return q, k, v, la, dO


def test_step_recurrence_equals_two_gla_passes():
    for seed in (1, 2):
        q, k, v, la, _ = _inputs(seed, T=11)
        assert np.allclose(gsa.gsa_fwd(q, k, v, la), gsa.two_pass_fwd(q, k, v, la),
                           rtol=1e-12, atol=1e-12)


def test_one_slot_is_gated_running_average():
    q, k, v, la, _ = _inputs(3, m=1)
    a = np.exp(la[:, 0])
    T = q.shape[0]
    ref = np.zeros((T, v.shape[1]))
    for t in range(T):
        for u in range(t + 1):
            ref[t] += (1.0 - a[u]) * np.prod(a[u + 1: t + 1]) * v[u]
    assert np.allclose(gsa.gsa_fwd(q, k, v, la), ref, rtol=1e-12, atol=1e-12)


def test_zero_queries_read_the_slot_mean():
    _, k, v, la, _ = _inputs(4)
    q = np.zeros((la.shape[0], k.shape[1]))
    a = np.exp(la)
    T, m = la.shape
    ref = np.zeros((T, v.shape[1]))
    for t in range(T):
        for j in range(m):
            Vj = np.zeros(v.shape[1])
            for u in range(t + 1):
                Vj += (1.0 - a[u, j]) * np.prod(a[u + 1: t + 1, j]) * v[u]
            ref[t] += Vj / m
    assert np.allclose(gsa.gsa_fwd(q, k, v, la), ref, rtol=1e-12, atol=1e-12)


def test_gradients_by_finite_differences():
    q, k, v, la, dO = _inputs(5, T=7)

    def loss(x):
        return float(np.sum(gsa.gsa_fwd(*x) * dO))

    grads = gsa.gsa_bwd(q, k, v, la, dO)
    base = [q, k, v, la]
    h = 1e-6
    for i, g in enumerate(grads):
        assert g.shape == base[i].shape
        for idx in [(0, 0), (3, 1), (base[i].shape[0] - 1, base[i].shape[1] - 1), (5, 2)]:
            xp = [x.copy() for x in base]
            xm = [x.copy() for x in base]
            xp[i][idx] += h
            xm[i][idx] -= h
            fd = (loss(xp) - loss(xm)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (i, idx, fd, g[idx])
