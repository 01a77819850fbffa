"""GPU parity of the scalar-gate variants (one gate per token and head, log_alpha
[B, H, T]; a constant decay per head as its data-independent case) against the oracle's
fp64 scalar layer (oracle/scalar.py): forward in both state modes, backward on both chunk
backward paths (bf16 chunk 64, and fp32 / chunk 128), gate logits, decode, gate cumsum."""
import numpy as np
import pytest

from gla_inputs import GlaConfig, generate
from oracle import gates, scalar
from tests.gpu_util import check, host, pick, say, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
TAU = 16.0


@pytest.fixture(scope="module")
def gla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_linear_rnn_amd as m
    m.lib()
    return m


def _inputs(d, dt, gate_name):
    out = {n: to_dev(d[n + "_store"], dt, DEV) for n in ("q", "k", "v", "dO") if n + "_store" in d}
    out["gate"] = to_dev(d[gate_name + "_store"], dt, DEV)
    return out


def _oracle(d, heads, gate_vals, logits, S0=None, dST=None, bwd=True):
    out = {k: [] for k in ("o", "S_T", "dq", "dk", "dv", "dla", "dS0")}
    for b, h in heads:
        s0 = None if S0 is None else S0[b, h].astype(np.float64)
        dst = None if dST is None else dST[b, h].astype(np.float64)
        x = gate_vals[b, h]
        la = gates.log_alpha_from_logits(x, TAU) if logits else x
        a = (d["q"][b, h], d["k"][b, h], d["v"][b, h], la)
        o, ST = scalar.scalar_fwd(*a, s0)
        out["o"].append(o)
        out["S_T"].append(ST)
        if bwd:
            dq, dk, dv, dla, dS0 = scalar.scalar_bwd(*a, d["dO"][b, h], s0, dst)
            if logits:
                dla = gates.logits_grad(dla, x, TAU)
            for kname, val in zip(("dq", "dk", "dv", "dla", "dS0"), (dq, dk, dv, dla, dS0)):
                out[kname].append(val)
    return {k: np.stack(v) for k, v in out.items() if v}


CASES = [
    # name, dtype, B, H, T, dk, dv, chunk, gate_mean, state mode, logits
    ("bf16_c64", "bf16", 2, 2, 300, 128, 128, 64, 0.0, "recompute", False),
    ("bf16_c64_mat_logits", "bf16", 1, 2, 200, 256, 64, 64, -3.0, "materialized", True),
    ("f32_ragged", "f32", 1, 2, 150, 64, 64, 64, 2.0, "recompute", False),
    ("bf16_c128_logits", "bf16", 1, 2, 257, 64, 128, 128, 0.0, "recompute", True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_scalar_fwd_bwd_small(gla, case):
    name, dt, B, H, T, dk, dv, C, gm, mode, logits = case
    cfg = GlaConfig(name=name, dtype=dt, B=B, H=H, T=T, dk=dk, dv=dv, chunk=C, gate_mean=gm)
    say(f"[scalar] {cfg} mode={mode} logits={logits}")
    d = generate(cfg)
    gname = "gate_logits_scalar" if logits else "log_alpha_scalar"
    x = _inputs(d, dt, gname)
    tau = TAU if logits else None
    rng = np.random.default_rng(6)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.5).astype(np.float32)
    dST = (rng.standard_normal((B, H, dk, dv)) * 0.5).astype(np.float32)
    S0d, dSTd = torch.from_numpy(S0).to(DEV), torch.from_numpy(dST).to(DEV)
    o, ST = gla.fwd(x["q"], x["k"], x["v"], x["gate"], S0d, chunk=C, state_mode=mode,
                    gate_tau=tau)
    g = gla.bwd(x["q"], x["k"], x["v"], x["gate"], x["dO"], S0d, dSTd, chunk=C, gate_tau=tau)
    torch.cuda.synchronize()
    assert tuple(g[3].shape) == (B, H, T)
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = _oracle(d, heads, d[gname], logits, S0, dST)
    check("o", pick(host(o), heads), ref["o"], dt)
    check("S_T", pick(host(ST), heads), ref["S_T"], dt)
    for kname, t in zip(("dq", "dk", "dv", "dla", "dS0"), g):
        check(kname, pick(host(t), heads), ref[kname], dt)


def test_constant_decay_per_head(gla):
    """RetNet-style: gamma_h = 1 - 2^-(5+h) for every token, no initial state."""
    B, H, T, dk, dv = 1, 4, 384, 128, 128
    cfg = GlaConfig(name="retnet", dtype="bf16", B=B, H=H, T=T, dk=dk, dv=dv, chunk=64)
    d = generate(cfg)
    gam = 1.0 - 2.0 ** -(5.0 + np.arange(H))
    la = np.broadcast_to(np.log(gam)[None, :, None], (B, H, T)).astype(np.float32)
    # bf16-representable values, so the device and the oracle see the same gates
    la_dev = torch.from_numpy(np.ascontiguousarray(la)).to(DEV).to(torch.bfloat16)
    la_exact = la_dev.to(torch.float64).cpu().numpy()
    x = _inputs(d, "bf16", "log_alpha_scalar")
    o, ST = gla.fwd(x["q"], x["k"], x["v"], la_dev)
    g = gla.bwd(x["q"], x["k"], x["v"], la_dev, x["dO"])
    torch.cuda.synchronize()
    heads = [(0, h) for h in range(H)]
    ref = _oracle(d, heads, la_exact, False)
    check("o", pick(host(o), heads), ref["o"], "bf16")
    check("S_T", pick(host(ST), heads), ref["S_T"], "bf16")
    for kname, t in zip(("dq", "dk", "dv", "dla"), g[:4]):
        check(kname, pick(host(t), heads), ref[kname], "bf16")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_scalar_decode_matches_oracle(gla, dt):
    B, H, T, dk, dv = 2, 2, 5, 128, 96
    cfg = GlaConfig(name="sdec", dtype=dt, B=B, H=H, T=T, dk=dk, dv=dv, chunk=64, seed=7)
    d = generate(cfg, with_dO=False)
    x = _inputs(d, dt, "gate_logits_scalar")
    rng = np.random.default_rng(8)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.5).astype(np.float32)
    S = torch.from_numpy(S0.copy()).to(DEV)
    o = gla.decode(x["q"], x["k"], x["v"], x["gate"], S, gate_tau=TAU)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = _oracle(d, heads, d["gate_logits_scalar"], True, S0, bwd=False)
    check("o", pick(host(o), heads), ref["o"], dt)
    # the state stays fp32 over the T steps: the fp32 bar
    check("S", pick(host(S), heads), ref["S_T"], "f32")


def test_scalar_gate_cumsum(gla):
    B, H, T, dk, C = 2, 3, 333, 128, 64
    cfg = GlaConfig(name="sgc", dtype="bf16", B=B, H=H, T=T, dk=dk, dv=64, chunk=C, seed=11)
    d = generate(cfg, with_dO=False)
    la = to_dev(d["log_alpha_scalar_store"], "bf16", DEV)
    g, gamma = gla.gate_cumsum(la, C, dk=dk)
    torch.cuda.synchronize()
    ref = np.zeros((B, H, T))
    for i0 in range(0, T, C):
        ref[..., i0:i0 + C] = np.cumsum(d["log_alpha_scalar"][..., i0:i0 + C], axis=-1)
    assert np.max(np.abs(host(g) - ref[..., None])) < 1e-5
    last = [min(T, i0 + C) - 1 for i0 in range(0, T, C)]
    assert np.max(np.abs(host(gamma) - ref[..., last][..., None])) < 1e-5


def test_scalar_full_size_sampled(gla):
    """The 1.3B-shape workload (B=4, H=4, T=2048, dk=256, dv=512) with scalar gates, in
    the launch configuration the benchmark uses; two heads checked against the oracle."""
    cfg = GlaConfig(name="gla1p3b_scalar", dtype="bf16", B=4, H=4, T=2048, dk=256, dv=512,
                    chunk=64)
    d = generate(cfg)
    x = _inputs(d, "bf16", "log_alpha_scalar")
    o, ST = gla.fwd(x["q"], x["k"], x["v"], x["gate"])
    g = gla.bwd(x["q"], x["k"], x["v"], x["gate"], x["dO"])
    torch.cuda.synchronize()
    heads = [(0, 0), (3, 2)]
    ref = _oracle(d, heads, d["log_alpha_scalar"], False)
    check("o", pick(host(o), heads), ref["o"], "bf16")
    for kname, t in zip(("dq", "dk", "dv", "dla"), g[:4]):
        check(kname, pick(host(t), heads), ref[kname], "bf16")
