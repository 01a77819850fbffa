"""The autograd wrappers (gla, gsa): their gradients are those of the direct entry points
(bit for bit: the same calls) and match the oracle on the same inputs; the gate options
pass through (gate logits, a scalar gate per token)."""
import numpy as np
import pytest

from gla_inputs import GlaConfig, generate, generate_gsa
from oracle import gates, gsa as ogsa, scalar
from tests.gpu_util import check, dev_inputs, host, oracle_heads, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def gla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_linear_rnn_amd as m
    m.lib()
    return m


def _leaf(t):
    return t.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gla_autograd(gla, dt):
    cfg = GlaConfig(name="ag", dtype=dt, B=1, H=2, T=200, dk=64, dv=128, chunk=64, seed=5)
    say(f"[autograd] {cfg}")
    d = generate(cfg)
    x = dev_inputs(d, dt, DEV)
    rng = np.random.default_rng(11)
    S0n = rng.standard_normal((1, 2, 64, 128)).astype(np.float32)
    dSTn = rng.standard_normal((1, 2, 64, 128)).astype(np.float32)
    S0, dST = torch.from_numpy(S0n).to(DEV), torch.from_numpy(dSTn).to(DEV)
    leaves = [_leaf(x[n]) for n in ("q", "k", "v", "log_alpha")] + [_leaf(S0)]
    o, S_T = gla.gla(*leaves)
    torch.autograd.backward([o, S_T], [x["dO"], dST])
    torch.cuda.synchronize()
    direct = gla.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["dO"], S0, dST)
    for name, leaf, ref in zip(("dq", "dk", "dv", "dla", "dS0"), leaves, direct):
        assert torch.equal(leaf.grad, ref), name
    heads = [(0, 0), (0, 1)]
    ref = oracle_heads(d, heads, S0n.astype(np.float64), dSTn.astype(np.float64))
    check("o", host(o)[0], ref["o"], dt)
    for name, leaf in zip(("dq", "dk", "dv", "dla", "dS0"), leaves):
        check(name, host(leaf.grad)[0], ref[name], dt)


def test_gla_autograd_gate_options(gla):
    """Gate logits (gate_tau) and a scalar gate per token through the autograd wrapper."""
    cfg = GlaConfig(name="ag_gates", dtype="f32", B=1, H=1, T=130, dk=64, dv=64, chunk=64, seed=6)
    d = generate(cfg)
    say(f"[autograd] gate options {cfg}")
    x = dev_inputs(d, "f32", DEV, names=("q", "k", "v", "dO", "gate_logits", "log_alpha_scalar"))
    leaves = [_leaf(x[n]) for n in ("q", "k", "v", "gate_logits")]
    o, _ = gla.gla(*leaves, gate_tau=16.0)
    o.backward(x["dO"])
    torch.cuda.synchronize()
    a = (d["q"][0, 0], d["k"][0, 0], d["v"][0, 0], d["gate_logits"][0, 0])
    o_ref, _ = gates.fwd_logits(*a, 16.0)
    check("o logits", host(o)[0, 0], o_ref, "f32")
    g_ref = gates.bwd_logits(*a, 16.0, d["dO"][0, 0])
    for name, leaf, r in zip(("dq", "dk", "dv", "dx"), leaves, g_ref):
        check(name + " logits", host(leaf.grad)[0, 0], r, "f32")
    leaves = [_leaf(x[n]) for n in ("q", "k", "v", "log_alpha_scalar")]
    o, _ = gla.gla(*leaves)
    o.backward(x["dO"])
    torch.cuda.synchronize()
    a = (d["q"][0, 0], d["k"][0, 0], d["v"][0, 0], d["log_alpha_scalar"][0, 0])
    o_ref, _ = scalar.scalar_fwd(*a)
    check("o scalar", host(o)[0, 0], o_ref, "f32")
    for name, leaf, r in zip(("dq", "dk", "dv", "dla"), leaves, scalar.scalar_bwd(*a, d["dO"][0, 0])):
        check(name + " scalar", host(leaf.grad)[0, 0], r, "f32")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gsa_autograd(gla, dt):
    cfg = GlaConfig(name="ag_gsa", dtype=dt, B=1, H=2, T=150, dk=64, dv=64, chunk=64, seed=7)
    say(f"[autograd] gsa {cfg}")
    d = generate_gsa(cfg, 64)
    x = {n: to_dev(d[n + "_store"], dt, DEV) for n in ("q", "k", "v", "dO", "log_alpha_slot")}
    leaves = [_leaf(x[n]) for n in ("q", "k", "v", "log_alpha_slot")]
    o = gla.gsa(*leaves)
    o.backward(x["dO"])
    torch.cuda.synchronize()
    direct = gla.gsa_bwd(x["q"], x["k"], x["v"], x["log_alpha_slot"], x["dO"])
    for name, leaf, ref in zip(("dq", "dk", "dv", "dla"), leaves, direct):
        assert torch.equal(leaf.grad, ref), name
    for h in range(2):
        a = (d["q"][0, h], d["k"][0, h], d["v"][0, h], d["log_alpha_slot"][0, h])
        check(f"o[{h}]", host(o)[0, h], ogsa.gsa_fwd(*a), dt)
        for name, leaf, r in zip(("dq", "dk", "dv", "dla"), leaves, ogsa.gsa_bwd(*a, d["dO"][0, h])):
            check(f"{name}[{h}]", host(leaf.grad)[0, h], r, dt)
