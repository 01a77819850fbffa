"""The training pair (gla_chunk_fwd_save / gla_chunk_bwd_saved, through ops.fwd_save /
ops.bwd_saved): the forward returns gla_chunk_fwd's bits (its later kernels read the high
parts of the kept transposed keys, the rounding gla_chunk_fwd stores) and the backward
from the saved intra-chunk operands gla_chunk_bwd's, and both match the oracle."""
import numpy as np
import pytest

from gla_inputs import CONFIGS, GlaConfig, generate
from tests.gpu_util import TOL, check, dev_inputs, host, oracle_heads, pick, say

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


CASES = [
    # name, dtype, B, H, T, dk, dv, chunk, gate option
    # five sequence segments of two chunks (ragged last), chained by the segment combine
    ("bf16_c64_seg5", "bf16", 1, 2, 600, 128, 128, 64, None),
    # two segments (the column tiles fill the chip's quota): one end-state scan
    ("bf16_c64_seg2", "bf16", 2, 4, 256, 64, 1024, 64, None),
    ("bf16_c128", "bf16", 1, 2, 333, 64, 128, 128, None),
    ("f32_c64", "f32", 1, 2, 200, 64, 128, 64, None),
    ("bf16_logits", "bf16", 1, 2, 300, 64, 128, 64, "logits"),
    ("bf16_scalar", "bf16", 1, 2, 300, 128, 64, 64, "scalar"),
]


def _run(gla, x, la, S0, dST, C, gate_tau):
    o, ST, sv = gla.fwd_save(x["q"], x["k"], x["v"], la, S0, chunk=C, gate_tau=gate_tau)
    o2, ST2 = gla.fwd(x["q"], x["k"], x["v"], la, S0, chunk=C, gate_tau=gate_tau)
    gs = gla.bwd_saved(x["q"], x["k"], x["v"], la, x["dO"], sv, S0, dST, chunk=C,
                       gate_tau=gate_tau)
    g = gla.bwd(x["q"], x["k"], x["v"], la, x["dO"], S0, dST, chunk=C, gate_tau=gate_tau)
    torch.cuda.synchronize()
    return o, ST, o2, ST2, gs, g


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_train_pair_small(gla, case):
    name, dt, B, H, T, dk, dv, C, opt = case
    say(f"[train pair] {name}")
    cfg = GlaConfig(name, dt, B, H, T, dk, dv, C, gate_mean=-0.5, seed=17)
    d = generate(cfg)
    names = ["q", "k", "v", "dO"]
    if opt == "logits":
        names.append("gate_logits")
    elif opt == "scalar":
        names.append("log_alpha_scalar")
    else:
        names.append("log_alpha")
    x = dev_inputs(d, dt, DEV, names=tuple(names))
    la = x[names[-1]]
    rng = np.random.default_rng(23)
    shp = (B, H, dk, dv)
    S0n = (rng.standard_normal(shp) * 0.5).astype(np.float32)
    dSTn = (rng.standard_normal(shp) * 0.5).astype(np.float32)
    S0, dST = torch.from_numpy(S0n).to(DEV), torch.from_numpy(dSTn).to(DEV)
    tau = 16.0 if opt == "logits" else None
    o, ST, o2, ST2, gs, g = _run(gla, x, la, S0, dST, C, tau)
    for nm, a, b in zip(("dq", "dk", "dv", "dla", "dS0"), gs, g):
        assert torch.equal(a, b), f"{name}: {nm} differs from gla_chunk_bwd"
    assert torch.equal(o, o2), f"{name}: o differs from gla_chunk_fwd"
    assert torch.equal(ST, ST2), f"{name}: S_T differs from gla_chunk_fwd"
    if opt is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
        ref = oracle_heads(d, heads, S0n.astype(np.float64), dSTn.astype(np.float64))
        got = {"o": o, "S_T": ST, "dq": gs[0], "dk": gs[1], "dv": gs[2], "dla": gs[3],
               "dS0": gs[4]}
        for k in ("o", "S_T", "dq", "dk", "dv", "dla", "dS0"):
            check(k, pick(host(got[k]), heads), ref[k], dt)


@pytest.mark.parametrize("name", ["gla1p3b_t2k", "gla340m_t2k", "sweep_t4096_c128"])
def test_train_pair_full_shape(gla, name):
    """The full workloads (the 1.3B and 340M head shapes at chunk 64, a chunk-128 sweep
    point): every head's output and gradients bit for bit those of gla_chunk_fwd and
    gla_chunk_bwd, one head against the oracle."""
    cfg = CONFIGS[name]
    say(f"[train pair] full shape {cfg}")
    d = generate(cfg)
    x = dev_inputs(d, cfg.dtype, DEV)
    o, ST, o2, ST2, gs, g = _run(gla, x, x["log_alpha"], None, None, cfg.chunk, None)
    for nm, a, b in zip(("dq", "dk", "dv", "dla", "dS0"), gs, g):
        assert torch.equal(a, b), f"{nm} differs from gla_chunk_bwd"
    assert torch.equal(o, o2) and torch.equal(ST, ST2), "forward differs from gla_chunk_fwd"
    heads = [(cfg.B - 1, cfg.H - 2)]
    ref = oracle_heads(d, heads)
    got = {"o": o, "dq": gs[0], "dk": gs[1], "dv": gs[2], "dla": gs[3]}
    for k in ("o", "dq", "dk", "dv", "dla"):
        check(k, pick(host(got[k]), heads), ref[k], cfg.dtype)


def test_train_pair_refusals(gla):
    """Materialized states have no saving forward; a short saved buffer is refused."""
    cfg = GlaConfig("tp_err", "bf16", 1, 1, 128, 64, 64, 64, seed=2)
    d = generate(cfg)
    x = dev_inputs(d, "bf16", DEV)
    desc = gla.make_desc(1, 1, 128, 64, 64, 64, 16, gla.BF16, gla.MATERIALIZED)
    with pytest.raises(gla.GlaError):
        gla.saved_bytes(desc)
    o, ST, sv = gla.fwd_save(x["q"], x["k"], x["v"], x["log_alpha"])
    with pytest.raises(ValueError):
        gla.bwd_saved(x["q"], x["k"], x["v"], x["log_alpha"], x["dO"], sv[:-256])
