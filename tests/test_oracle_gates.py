"""Pins of the oracle's gate front-end (oracle/gates.py) against facts that do not come
from it: the textbook definition of logsigmoid where it is accurate, its asymptotes, the
derivative by finite differences, the whole layer's gradient with respect to the logits
by finite differences, and the ungated limit (causal linear attention by numpy matmul)."""
import numpy as np

from oracle import gates
from oracle.recurrence import recurrence_fwd


def test_logsigmoid_matches_definition_where_direct_is_accurate():
    # for x above a few units 1 + e^-x rounds off in the direct form; that tail is pinned
    # by the asymptote below
    x = np.linspace(-20, 4, 2401)
    direct = np.log(1.0 / (1.0 + np.exp(-x)))
    assert np.max(np.abs(gates.logsigmoid(x) - direct) / np.abs(direct)) < 1e-13


def test_logsigmoid_asymptotes_and_value_at_zero():
    assert gates.logsigmoid(0.0) == -np.log(2.0)
    for x in (-50.0, -300.0, -700.0):      # log sigmoid(x) = x - log(1 + e^x) -> x
        assert abs(gates.logsigmoid(x) - x) <= 1e-20 + 2e-16 * abs(x)
    for x in (30.0, 40.0, 60.0):           # log sigmoid(x) = -log(1 + e^-x) -> -e^-x
        assert abs(gates.logsigmoid(x) / -np.exp(-x) - 1.0) < 1e-12
    assert np.all(np.isfinite(gates.logsigmoid(np.array([-1e4, 1e4]))))


def test_sigmoid_neg_definition_and_symmetry():
    x = np.linspace(-30, 30, 601)
    assert np.allclose(gates.sigmoid_neg(x), 1.0 / (1.0 + np.exp(x)), rtol=1e-14, atol=0)
    # sigmoid(x) + sigmoid(-x) = 1
    assert np.allclose(gates.sigmoid_neg(-x) + gates.sigmoid_neg(x), 1.0, rtol=0, atol=1e-15)
    assert gates.sigmoid_neg(1e4) == 0.0 and gates.sigmoid_neg(-1e4) == 1.0


def test_logsigmoid_derivative_by_finite_differences():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(200) * 4
    h = 1e-6
    fd = (gates.logsigmoid(x + h) - gates.logsigmoid(x - h)) / (2 * h)
    assert np.max(np.abs(fd - gates.sigmoid_neg(x))) < 1e-8


def test_layer_gradient_wrt_logits_by_finite_differences():
    rng = np.random.default_rng(5)
    T, dk, dv, tau = 6, 3, 3, 4.0
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    v, dO = rng.standard_normal((T, dv)), rng.standard_normal((T, dv))
    x = rng.standard_normal((T, dk)) * 2
    S0, dST = rng.standard_normal((dk, dv)), rng.standard_normal((dk, dv))

    def loss(xx):
        o, ST = gates.fwd_logits(q, k, v, xx, tau, S0)
        return float(np.sum(o * dO) + np.sum(ST * dST))

    _, _, _, dx, _ = gates.bwd_logits(q, k, v, x, tau, dO, S0, dST)
    h = 1e-6
    for t, d in [(0, 0), (2, 1), (5, 2), (3, 0), (4, 2)]:
        xp, xm = x.copy(), x.copy()
        xp[t, d] += h
        xm[t, d] -= h
        fd = (loss(xp) - loss(xm)) / (2 * h)
        assert abs(fd - dx[t, d]) < 1e-7, (t, d, fd, dx[t, d])


def test_open_gates_reduce_to_causal_linear_attention():
    """Very large logits give alpha = 1 to double precision: plain causal linear
    attention, tril(Q K^T) V + Q S0, computed with numpy matmul."""
    rng = np.random.default_rng(9)
    T, dk, dv = 12, 4, 5
    q, k, v = (rng.standard_normal((T, d)) for d in (dk, dk, dv))
    S0 = rng.standard_normal((dk, dv))
    x = np.full((T, dk), 60.0)
    o, ST = gates.fwd_logits(q, k, v, x, 16.0, S0)
    ref = np.tril(q @ k.T) @ v + q @ S0
    assert np.max(np.abs(o - ref)) < 1e-10
    assert np.max(np.abs(ST - (S0 + k.T @ v))) < 1e-10
    # and the gate is what the layer sees through recurrence_fwd
    o2, _ = recurrence_fwd(q, k, v, gates.log_alpha_from_logits(x, 16.0), S0)
    assert np.array_equal(o, o2)
