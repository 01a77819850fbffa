"""Pins for the fp64 oracle: each check compares it with something it does not compute
itself (a closed form, a BLAS product, finite differences, torch autograd on an
independent graph, exact rational arithmetic, an invariance the mathematics fixes)."""
from fractions import Fraction
import math

import numpy as np
import pytest

from oracle import recurrence_fwd, recurrence_bwd, quadratic_fwd, closed_form_gate_grad
from oracle import chunkwise
from oracle.compare import max_rel, normwise


def _case(rng, B=2, H=2, T=23, dk=6, dv=5, la_scale=0.4, S0=True, dST=True):
    q = rng.standard_normal((B, H, T, dk)) * 0.6
    k = rng.standard_normal((B, H, T, dk)) * 0.6
    v = rng.standard_normal((B, H, T, dv))
    la = -np.abs(rng.standard_normal((B, H, T, dk))) * la_scale
    dO = rng.standard_normal((B, H, T, dv))
    s0 = rng.standard_normal((B, H, dk, dv)) if S0 else None
    dst = rng.standard_normal((B, H, dk, dv)) if dST else None
    return q, k, v, la, dO, s0, dst


# P1: step recurrence == quadratic (parallel) form -----------------------------------
@pytest.mark.parametrize("T,dk,dv", [(1, 3, 2), (17, 4, 7), (64, 8, 8)])
def test_fwd_matches_quadratic_form(rng, T, dk, dv):
    q, k, v, la, _, s0, _ = _case(rng, T=T, dk=dk, dv=dv)
    o, _ = recurrence_fwd(q, k, v, la, s0)
    assert max_rel(o, quadratic_fwd(q, k, v, la, s0)) < 1e-12
    o0, _ = recurrence_fwd(q, k, v, la)
    assert max_rel(o0, quadratic_fwd(q, k, v, la)) < 1e-12


# P2: alpha = 1 reduces to causal linear attention (numpy matmul / BLAS) -------------
def test_ungated_is_causal_linear_attention(rng):
    q, k, v, la, dO, s0, dst = _case(rng, T=29, dk=7, dv=9)
    la = np.zeros_like(la)
    o, ST = recurrence_fwd(q, k, v, la, s0)
    W = np.tril(q @ np.swapaxes(k, -1, -2))
    assert max_rel(o, W @ v + q @ s0) < 1e-12
    assert max_rel(ST, np.swapaxes(k, -1, -2) @ v + s0) < 1e-12
    dq, dk, dv, dla, dS0 = recurrence_bwd(q, k, v, la, dO, s0, dst)
    P = np.tril(dO @ np.swapaxes(v, -1, -2))           # dO_t . v_s for s <= t
    assert max_rel(dq, P @ k + dO @ np.swapaxes(s0, -1, -2)) < 1e-12
    assert max_rel(dk, np.swapaxes(P, -1, -2) @ q + v @ np.swapaxes(dst, -1, -2)) < 1e-12
    assert max_rel(dv, np.swapaxes(W, -1, -2) @ dO + k @ dst) < 1e-12
    assert max_rel(dS0, np.swapaxes(q, -1, -2) @ dO + dst) < 1e-12


# P3: state carry, forward and backward ------------------------------------------
@pytest.mark.parametrize("split", [1, 11, 22])
def test_chaining(rng, split):
    q, k, v, la, dO, s0, dst = _case(rng, T=23)
    o, ST = recurrence_fwd(q, k, v, la, s0)
    sl1, sl2 = slice(0, split), slice(split, None)
    o1, S1 = recurrence_fwd(q[..., sl1, :], k[..., sl1, :], v[..., sl1, :], la[..., sl1, :], s0)
    o2, S2 = recurrence_fwd(q[..., sl2, :], k[..., sl2, :], v[..., sl2, :], la[..., sl2, :], S1)
    assert max_rel(np.concatenate([o1, o2], -2), o) < 1e-12
    assert max_rel(S2, ST) < 1e-12
    full = recurrence_bwd(q, k, v, la, dO, s0, dst)
    g2 = recurrence_bwd(q[..., sl2, :], k[..., sl2, :], v[..., sl2, :], la[..., sl2, :],
                        dO[..., sl2, :], S1, dst)
    g1 = recurrence_bwd(q[..., sl1, :], k[..., sl1, :], v[..., sl1, :], la[..., sl1, :],
                        dO[..., sl1, :], s0, g2[4])
    for i in range(4):
        assert max_rel(np.concatenate([g1[i], g2[i]], -2), full[i]) < 1e-12
    assert max_rel(g1[4], full[4]) < 1e-12


# P4: finite differences on every gradient -------------------------------------------
def _loss(q, k, v, la, s0, dO, dst):
    o, ST = recurrence_fwd(q, k, v, la, s0)
    return float(np.sum(o * dO) + np.sum(ST * dst))


def test_gradients_match_finite_differences(rng):
    q, k, v, la, dO, s0, dst = _case(rng, B=1, H=2, T=9, dk=3, dv=4)
    grads = recurrence_bwd(q, k, v, la, dO, s0, dst)
    args = [q, k, v, la, s0]
    h = 1e-6
    names = ["q", "k", "v", "la", "S0"]
    got = list(grads[:4]) + [grads[4]]
    for ai, (name, gr) in enumerate(zip(names, got)):
        base = args[ai]
        fd = np.zeros_like(base)
        it = np.nditer(base, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[ai][idx] += h
            xm[ai][idx] -= h
            fd[idx] = (_loss(*xp, dO, dst) - _loss(*xm, dO, dst)) / (2 * h)
        assert np.max(np.abs(fd - gr)) < 1e-7, name


# torch autograd on an independently written fp64 graph ----------------------------
def test_gradients_match_torch_autograd(rng):
    torch = pytest.importorskip("torch")
    q, k, v, la, dO, s0, dst = _case(rng, B=2, H=1, T=31, dk=5, dv=3)
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for n, a in dict(q=q, k=k, v=v, la=la, s0=s0).items()}
    S = t["s0"]
    outs = []
    for i in range(q.shape[-2]):
        S = torch.exp(t["la"][..., i, :]).unsqueeze(-1) * S + \
            t["k"][..., i, :].unsqueeze(-1) * t["v"][..., i, :].unsqueeze(-2)
        outs.append(torch.einsum("bhd,bhdv->bhv", t["q"][..., i, :], S))
    o = torch.stack(outs, dim=-2)
    loss = (o * torch.tensor(dO)).sum() + (S * torch.tensor(dst)).sum()
    loss.backward()
    dq, dk, dv, dla, dS0 = recurrence_bwd(q, k, v, la, dO, s0, dst)
    for mine, name in [(dq, "q"), (dk, "k"), (dv, "v"), (dla, "la"), (dS0, "s0")]:
        assert max_rel(mine, t[name].grad.numpy()) < 1e-12, name


# P5: the pages' closed-form gate gradient equals the direct one ------------------------
@pytest.mark.parametrize("with_state", [False, True])
def test_closed_form_gate_gradient(rng, with_state):
    q, k, v, la, dO, s0, dst = _case(rng, T=41, S0=with_state, dST=with_state)
    dq, dk, dv, dla, _ = recurrence_bwd(q, k, v, la, dO, s0, dst)
    _, ST = recurrence_fwd(q, k, v, la, s0)
    cf = closed_form_gate_grad(q, dq, k, dk, ST if with_state else None, dst)
    assert max_rel(cf, dla) < 1e-12
    if with_state:   # dropping the final-state term must be detected
        cf_bad = closed_form_gate_grad(q, dq, k, dk)
        assert max_rel(cf_bad, dla) > 1e-3


# P6: chunkwise form == recurrence for any chunk / sub-chunk size ---------------------
@pytest.mark.parametrize("C,c", [(1, 1), (16, 1), (16, 4), (16, 16), (64, 16), (128, 16),
                                 (50, 16), (200, 200)])
def test_chunkwise_matches_recurrence(rng, C, c):
    q, k, v, la, dO, s0, dst = _case(rng, B=1, H=2, T=150, dk=6, dv=5, la_scale=0.8)
    o, ST = recurrence_fwd(q, k, v, la, s0)
    oc, STc, _ = chunkwise.chunkwise_fwd(q, k, v, la, s0, C=C, c=c)
    assert max_rel(oc, o) < 1e-12 and max_rel(STc, ST) < 1e-12
    ref = recurrence_bwd(q, k, v, la, dO, s0, dst)
    got = chunkwise.chunkwise_bwd(q, k, v, la, dO, s0, dst, C=C, c=c)
    for i, n in enumerate(["dq", "dk", "dv", "dla", "dS0"]):
        assert max_rel(got[i], ref[i]) < 1e-11, n


def test_chunkwise_intermediates(rng):
    """g is the chunk-local cumsum; states are the recurrence's states at chunk starts."""
    q, k, v, la, dO, s0, dst = _case(rng, B=1, H=1, T=40, dk=3, dv=2)
    _, _, it = chunkwise.chunkwise_fwd(q, k, v, la, s0, C=16, c=4)
    g = it["g"]
    assert np.allclose(g[..., 16, :], la[..., 16, :]) and np.allclose(g[..., 0, :], la[..., 0, :])
    assert np.allclose(g[..., 39, :], la[..., 32:40, :].sum(-2))
    assert np.allclose(it["gamma"][..., 2, :], la[..., 32:40, :].sum(-2))
    for i, t0 in enumerate([0, 16, 32]):
        if t0 == 0:
            ref = s0
        else:
            _, ref = recurrence_fwd(q[..., :t0, :], k[..., :t0, :], v[..., :t0, :],
                                    la[..., :t0, :], s0)
        assert max_rel(it["states"][..., i, :, :], ref) < 1e-12
    # A below the diagonal equals the quadratic weights restricted to the chunk
    A = it["A"][0, 0, 1]
    L = np.cumsum(la[0, 0, 16:32], axis=0)
    for t in range(16):
        for s in range(16):
            w = np.sum(q[0, 0, 16 + t] * k[0, 0, 16 + s] * np.exp(L[t] - L[s])) if s <= t else 0.0
            assert abs(A[t, s] - w) < 1e-12


# P7: closed forms and invariants ---------------------------------------------------
def test_single_step_closed_form(rng):
    q, k, v, la, _, s0, _ = _case(rng, T=1, dk=4, dv=3)
    o, ST = recurrence_fwd(q, k, v, la, s0)
    qk = np.sum(q[..., 0, :] * k[..., 0, :], -1)[..., None]
    ref = qk * v[..., 0, :] + ((q[..., 0, :] * np.exp(la[..., 0, :]))[..., None, :] @ s0)[..., 0, :]
    assert max_rel(o[..., 0, :], ref) < 1e-14


def test_vanishing_gate_keeps_only_current_token(rng):
    q, k, v, la, _, _, _ = _case(rng, T=12)
    la = np.full_like(la, -60.0)
    o, _ = recurrence_fwd(q, k, v, la)
    ref = np.sum(q * k, -1)[..., None] * v
    # alpha = exp(-60) ~ 1e-26: what is left of the past is far below fp64 rounding
    assert max_rel(o, ref) < 1e-14


def test_value_scaling(rng):
    q, k, v, la, dO, _, _ = _case(rng, T=19, S0=False, dST=False)
    s = 2.5
    a = recurrence_bwd(q, k, v, la, dO)
    b = recurrence_bwd(q, k, s * v, la, dO)
    o1, _ = recurrence_fwd(q, k, v, la)
    o2, _ = recurrence_fwd(q, k, s * v, la)
    assert max_rel(o2, s * o1) < 1e-13
    for i in (0, 1, 3):
        assert max_rel(b[i], s * a[i]) < 1e-13
    assert max_rel(b[2], a[2]) < 1e-13


def test_exact_rational_scalar_example():
    """dk = dv = 1, two key dims collapsed to scalars: the recurrence by hand in exact
    rational arithmetic."""
    alphas = [Fraction(1, 2), Fraction(3, 4), Fraction(1, 8), Fraction(7, 8), Fraction(1, 1)]
    qs = [Fraction(1), Fraction(-2), Fraction(3, 2), Fraction(1, 3), Fraction(5)]
    ks = [Fraction(2), Fraction(1, 2), Fraction(-1), Fraction(4), Fraction(1, 5)]
    vs = [Fraction(3), Fraction(-1), Fraction(2), Fraction(1, 2), Fraction(-3)]
    s = Fraction(1, 3)
    exact = []
    for a, qq, kk, vv in zip(alphas, qs, ks, vs):
        s = a * s + kk * vv
        exact.append(qq * s)
    f = lambda xs: np.array([float(x) for x in xs]).reshape(1, 1, -1, 1)
    la = np.log(f(alphas))
    o, ST = recurrence_fwd(f(qs), f(ks), f(vs), la, np.array([[[[1 / 3]]]]))
    assert np.allclose(o.ravel(), [float(x) for x in exact], rtol=1e-14, atol=0)
    assert abs(ST.ravel()[0] - float(s)) < 1e-14


def test_golden_fixture():
    """Regression pin: the tiny case stored in tests/golden by make_golden.py."""
    import json, os
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_case.json")
    with open(path) as fh:
        gd = json.load(fh)
    arr = {k: np.array(v, dtype=np.float64) for k, v in gd["arrays"].items()}
    o, ST = recurrence_fwd(arr["q"], arr["k"], arr["v"], arr["log_alpha"], arr["S0"])
    assert max_rel(o, arr["o"]) < 1e-13 and max_rel(ST, arr["S_T"]) < 1e-13
    g = recurrence_bwd(arr["q"], arr["k"], arr["v"], arr["log_alpha"], arr["dO"], arr["S0"],
                       arr["dS_T"])
    for i, n in enumerate(["dq", "dk", "dv", "dlog_alpha", "dS0"]):
        assert max_rel(g[i], arr[n]) < 1e-13, n


def test_compare_metrics():
    y = np.array([1.0, -2.0, 0.0, 4.0])
    x = y + np.array([0.1, 0.0, 0.0, -0.2])
    assert math.isclose(max_rel(x, y), 0.2 / 4.0)
    assert math.isclose(normwise(x, y), math.sqrt(0.05) / math.sqrt(21.0))
