"""GPU parity of the gate front-end (gates given as logits x, log_alpha = logsigmoid(x) /
tau formed inside the kernels, dlog_alpha returned as the gradient with respect to x)
against the oracle's fp64 front-end and chain rule."""
import numpy as np
import pytest

from gla_inputs import CONFIGS, GlaConfig, generate
from oracle import gates
from tests.gpu_util import check, host, pick, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TAU = 16.0
DEV = "cuda:0"


@pytest.fixture(scope="module")
def gla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_linear_rnn_amd as m
    m.lib()
    return m


def _inputs(d, dt):
    return {n: to_dev(d[n + "_store"], dt, DEV) for n in ("q", "k", "v", "gate_logits", "dO")
            if n + "_store" in d}


def _oracle(d, heads, S0=None, dST=None):
    out = {k: [] for k in ("o", "S_T", "dq", "dk", "dv", "dx", "dS0")}
    for b, h in heads:
        s0 = None if S0 is None else S0[b, h].astype(np.float64)
        dst = None if dST is None else dST[b, h].astype(np.float64)
        a = (d["q"][b, h], d["k"][b, h], d["v"][b, h], d["gate_logits"][b, h], TAU)
        o, ST = gates.fwd_logits(*a, s0)
        out["o"].append(o)
        out["S_T"].append(ST)
        if "dO" in d:
            g = gates.bwd_logits(*a, d["dO"][b, h], s0, dst)
            for kname, val in zip(("dq", "dk", "dv", "dx", "dS0"), g):
                out[kname].append(val)
    return {k: np.stack(v) for k, v in out.items() if v}


CASES = [
    # name, dtype, B, H, T, dk, dv, chunk, gate_mean, mode
    ("f32_ragged", "f32", 1, 2, 150, 64, 64, 64, 0.0, "recompute"),
    ("bf16_c64_mat", "bf16", 2, 1, 200, 128, 64, 64, -3.0, "materialized"),
    ("bf16_c128", "bf16", 1, 2, 257, 64, 128, 128, 2.0, "recompute"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_logits_fwd_bwd_small(gla, case):
    name, dt, B, H, T, dk, dv, C, gm, mode = case
    cfg = GlaConfig(name=name, dtype=dt, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C, gate_mean=gm)
    say(f"[gates] {cfg} mode={mode}")
    d = generate(cfg)
    x = _inputs(d, dt)
    rng = np.random.default_rng(4)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.5).astype(np.float32)
    dST = (rng.standard_normal((B, H, dk, dv)) * 0.5).astype(np.float32)
    S0d, dSTd = torch.from_numpy(S0).to(DEV), torch.from_numpy(dST).to(DEV)
    o, ST = gla.fwd(x["q"], x["k"], x["v"], x["gate_logits"], S0d, chunk=C, state_mode=mode,
                    gate_tau=TAU)
    g = gla.bwd(x["q"], x["k"], x["v"], x["gate_logits"], x["dO"], S0d, dSTd, chunk=C,
                gate_tau=TAU)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = _oracle(d, heads, S0, dST)
    check("o", pick(host(o), heads), ref["o"], dt)
    check("S_T", pick(host(ST), heads), ref["S_T"], dt)
    for kname, t in zip(("dq", "dk", "dv", "dx", "dS0"), g):
        check(kname, pick(host(t), heads), ref[kname], dt)


def test_logits_full_size_sampled_heads(gla):
    cfg = CONFIGS["gla1p3b_t2k"]
    heads = [(1, 2)]
    d = generate(cfg)
    x = _inputs(d, cfg.dtype)
    o, ST = gla.fwd(x["q"], x["k"], x["v"], x["gate_logits"], gate_tau=TAU)
    g = gla.bwd(x["q"], x["k"], x["v"], x["gate_logits"], x["dO"], gate_tau=TAU)
    torch.cuda.synchronize()
    ref = _oracle(d, heads)
    check("o", pick(host(o), heads), ref["o"], cfg.dtype)
    check("S_T", pick(host(ST), heads), ref["S_T"], cfg.dtype)
    for kname, t in zip(("dq", "dk", "dv", "dx", "dS0"), g):
        check(kname, pick(host(t), heads), ref[kname], cfg.dtype)


def test_logits_decode_and_gate_cumsum(gla):
    cfg = GlaConfig(name="gate_dec", dtype="bf16", B=2, H=2, T=8, dk=96, dv=64, chunk=64,
                    gate_mean=0.0, bwd=False)
    d = generate(cfg, with_dO=False)
    x = _inputs(d, "bf16")
    S0 = (np.random.default_rng(2).standard_normal((2, 2, 96, 64)) * 0.5).astype(np.float32)
    S = torch.from_numpy(S0.copy()).to(DEV)
    o = gla.decode(x["q"], x["k"], x["v"], x["gate_logits"], S, gate_tau=TAU)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(2) for h in range(2)]
    ref = _oracle(d, heads, S0)
    check("o decode", pick(host(o), heads), ref["o"], "bf16")
    check("S decode", pick(host(S), heads), ref["S_T"], "f32")
    # the gate cumsum kernel applies the same front-end
    cfg2 = GlaConfig(name="gate_cs", dtype="f32", B=1, H=2, T=150, dk=64, dv=64, chunk=64,
                     bwd=False)
    d2 = generate(cfg2, with_dO=False)
    la_d = to_dev(d2["gate_logits_store"], "f32", DEV)
    g, gamma = gla.gate_cumsum(la_d, chunk=64, gate_tau=TAU)
    torch.cuda.synchronize()
    la = gates.log_alpha_from_logits(d2["gate_logits"], TAU)
    ref_g = np.zeros_like(la)
    for i in range(0, 150, 64):
        ref_g[:, :, i:i + 64] = np.cumsum(la[:, :, i:i + 64], axis=2)
    check("g", host(g), ref_g, "f32")
    check("gamma", host(gamma)[:, :, -1], ref_g[:, :, -1], "f32")
