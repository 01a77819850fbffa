"""GPU parity of the recurrent (decoding) entry point gla_decode against the fp64
oracle's step recurrence, and its consistency with the chunkwise forward.

The decode call runs T tokens in order with the float32 state updated in place, so its
definition is exactly the oracle's step recurrence with S0 = the state on entry."""
import numpy as np
import pytest

from gla_inputs import GlaConfig, generate
from oracle import recurrence_fwd
from tests.gpu_util import TOL, check, dev_inputs, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def gla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_linear_rnn_amd as m
    m.lib()
    return m


DEV = "cuda:0"

CASES = [
    # name, dtype, B, H, T, dk, dv, gate_mean
    ("f32_one_token", "f32", 2, 3, 1, 64, 96, 0.0),
    ("f32_dk32_dv32", "f32", 1, 2, 7, 32, 32, 0.0),
    ("bf16_one_token_1p3b", "bf16", 2, 4, 1, 256, 512, 0.0),
    ("bf16_dk96_tokens", "bf16", 2, 2, 9, 96, 64, -3.0),
    ("bf16_dk224_slow", "bf16", 1, 2, 16, 224, 160, 2.0),
]


def _state(B, H, dk, dv, seed=11, scale=0.5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, dk, dv)) * scale).astype(np.float32)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(gla, case):
    name, dt, B, H, T, dk, dv, gm = case
    cfg = GlaConfig(name=name, dtype=dt, B=B, H=H, T=T, dk=dk, dv=dv, chunk=64, gate_mean=gm,
                    bwd=False)
    say(f"[decode] {cfg}")
    d = generate(cfg, with_dO=False)
    x = dev_inputs(d, dt, DEV, names=("q", "k", "v", "log_alpha"))
    S0 = _state(B, H, dk, dv)
    S = torch.from_numpy(S0.copy()).to(DEV)
    o = gla.decode(x["q"], x["k"], x["v"], x["log_alpha"], S)
    torch.cuda.synchronize()
    ref_o = np.empty((B, H, T, dv))
    ref_S = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            ref_o[b, h], ref_S[b, h] = recurrence_fwd(d["q"][b, h], d["k"][b, h], d["v"][b, h],
                                                      d["log_alpha"][b, h],
                                                      S0[b, h].astype(np.float64))
    check("o", host(o), ref_o, dt)
    # the state is float32 for either input type
    check("S", host(S), ref_S, "f32")


def test_one_call_equals_token_by_token(gla):
    """T tokens in one call and T calls of one token do the same fp32 arithmetic."""
    cfg = GlaConfig(name="dec_chain", dtype="bf16", B=2, H=2, T=64, dk=128, dv=128, chunk=64,
                    bwd=False)
    d = generate(cfg, with_dO=False)
    x = dev_inputs(d, "bf16", DEV, names=("q", "k", "v", "log_alpha"))
    S0 = torch.from_numpy(_state(2, 2, 128, 128)).to(DEV)
    S1 = S0.clone()
    o1 = gla.decode(x["q"], x["k"], x["v"], x["log_alpha"], S1)
    S2 = S0.clone()
    outs = []
    for t in range(cfg.T):
        sl = slice(t, t + 1)
        outs.append(gla.decode(*(x[n][:, :, sl].contiguous() for n in ("q", "k", "v", "log_alpha")),
                               S2))
    o2 = torch.cat(outs, dim=2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(S1, S2)


def test_decode_agrees_with_chunk_forward(gla):
    """Prefix by the chunkwise forward, then the same tokens by decoding, from one S0."""
    cfg = GlaConfig(name="dec_vs_chunk", dtype="bf16", B=1, H=2, T=192, dk=256, dv=512,
                    chunk=64, bwd=False)
    d = generate(cfg, with_dO=False)
    x = dev_inputs(d, "bf16", DEV, names=("q", "k", "v", "log_alpha"))
    S0 = _state(1, 2, 256, 512)
    o_c, ST_c = gla.fwd(x["q"], x["k"], x["v"], x["log_alpha"], torch.from_numpy(S0).to(DEV))
    S = torch.from_numpy(S0.copy()).to(DEV)
    o_d = gla.decode(x["q"], x["k"], x["v"], x["log_alpha"], S)
    torch.cuda.synchronize()
    ref_o, ref_S = recurrence_fwd(d["q"][0, 1], d["k"][0, 1], d["v"][0, 1], d["log_alpha"][0, 1],
                                  S0[0, 1].astype(np.float64))
    check("o decode", host(o_d)[0, 1], ref_o, "bf16")
    check("o chunk", host(o_c)[0, 1], ref_o, "bf16")
    check("S decode", host(S)[0, 1], ref_S, "f32")
    check("S chunk", host(ST_c)[0, 1], ref_S, "bf16")
    check("o decode vs chunk", host(o_d), host(o_c), "bf16")


def test_empty_calls_leave_the_state(gla):
    S0 = torch.from_numpy(_state(1, 2, 64, 64)).to(DEV)
    S = S0.clone()
    z = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    o = gla.decode(z, z, z, z, S)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 64)
    assert torch.equal(S, S0)
    zb = torch.empty((0, 2, 1, 64), dtype=torch.bfloat16, device=DEV)
    gla.decode(zb, zb, zb, zb, torch.empty((0, 2, 64, 64), device=DEV))


def test_decode_invalid_arguments(gla):
    q = torch.zeros((1, 1, 1, 48), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device=DEV)
    S = torch.zeros((1, 1, 48, 64), device=DEV)
    with pytest.raises(gla.GlaError):
        gla.decode(q, q, v, q, S)                   # dk = 48: not a multiple of 32
    q64 = torch.zeros((1, 1, 1, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        gla.decode(q64, q64, v, q64, torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16,
                                                  device=DEV))   # state must be float32
    tol = TOL["bf16"]
    assert tol["normwise"] == 5e-3
