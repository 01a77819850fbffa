"""GPU parity of Gated Slot Attention (gla_gsa_fwd / gla_gsa_bwd, float32 and bfloat16)
against the oracle's slot recurrence and its fp64 autograd gradient (oracle/gsa.py) on the
same (rounded) inputs: ragged chunks, 128 slots, a single token, a long thin head, the
empty problem, and the 1.3B head shape with 64 slots (sampled heads)."""
import numpy as np
import pytest

from gla_inputs import GlaConfig, generate_gsa
from oracle import gsa
from tests.gpu_util import check, host, say, to_dev

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


def _dev(d, dt="f32"):
    return {n: to_dev(d[n + "_store"], dt, DEV) for n in ("q", "k", "v", "dO", "log_alpha_slot")}


CASES = [
    # name, B, H, T, dk, dv, slots, gate_mean
    ("ragged", 1, 2, 150, 64, 64, 64, 0.0),
    ("dk128_dv192", 2, 1, 200, 128, 192, 64, 2.0),
    ("slots128", 1, 1, 130, 64, 128, 128, -3.0),
    ("one_token", 1, 1, 1, 64, 64, 64, 0.0),
    # 33 chunks of one head: the key-slot scans (forward and reverse) in 4 segments walked
    # from their chained start states, ragged last chunk
    ("thin_long", 1, 1, 2100, 64, 64, 64, -1.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gsa_fwd_bwd_small(gla, case):
    name, B, H, T, dk, dv, m, gm = case
    cfg = GlaConfig(name=name, dtype="f32", B=B, H=H, T=T, dk=dk, dv=dv, chunk=64, gate_mean=gm)
    say(f"[gsa] {cfg} slots={m}")
    d = generate_gsa(cfg, m)
    x = _dev(d)
    o = gla.gsa_fwd(x["q"], x["k"], x["v"], x["log_alpha_slot"])
    g = gla.gsa_bwd(x["q"], x["k"], x["v"], x["log_alpha_slot"], x["dO"])
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            a = (d["q"][b, h], d["k"][b, h], d["v"][b, h], d["log_alpha_slot"][b, h])
            check(f"o[{b},{h}]", host(o)[b, h], gsa.gsa_fwd(*a), "f32")
            ref = gsa.gsa_bwd(*a, d["dO"][b, h])
            for kname, t, r in zip(("dq", "dk", "dv", "dla"), g, ref):
                check(f"{kname}[{b},{h}]", host(t)[b, h], r, "f32")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_gsa_bf16_small(gla, case):
    """bf16 inputs and outputs (first pass in fp32, second pass on the layer's bf16 path),
    against the oracle on the same bf16-rounded inputs, at the bf16 tolerances."""
    name, B, H, T, dk, dv, m, gm = case
    cfg = GlaConfig(name=name, dtype="bf16", B=B, H=H, T=T, dk=dk, dv=dv, chunk=64,
                    gate_mean=gm)
    say(f"[gsa bf16] {cfg} slots={m}")
    d = generate_gsa(cfg, m)
    x = _dev(d, "bf16")
    o = gla.gsa_fwd(x["q"], x["k"], x["v"], x["log_alpha_slot"])
    g = gla.gsa_bwd(x["q"], x["k"], x["v"], x["log_alpha_slot"], x["dO"])
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16 and all(t.dtype == torch.bfloat16 for t in g)
    for b in range(B):
        for h in range(H):
            a = (d["q"][b, h], d["k"][b, h], d["v"][b, h], d["log_alpha_slot"][b, h])
            check(f"o[{b},{h}]", host(o)[b, h], gsa.gsa_fwd(*a), "bf16")
            ref = gsa.gsa_bwd(*a, d["dO"][b, h])
            for kname, t, r in zip(("dq", "dk", "dv", "dla"), g, ref):
                check(f"{kname}[{b},{h}]", host(t)[b, h], r, "bf16")


def test_gsa_bf16_full_size_sampled(gla):
    """bf16 at B=4, H=4, dk=256, dv=512, 64 slots: forward and backward of two sampled heads
    of a T=512 run."""
    cfg = GlaConfig(name="gsa1p3b_bf16_t512", dtype="bf16", B=4, H=4, T=512, dk=256, dv=512,
                    chunk=64)
    say(f"[gsa bf16] {cfg}")
    d = generate_gsa(cfg, 64)
    x = _dev(d, "bf16")
    o = gla.gsa_fwd(x["q"], x["k"], x["v"], x["log_alpha_slot"])
    g = gla.gsa_bwd(x["q"], x["k"], x["v"], x["log_alpha_slot"], x["dO"])
    torch.cuda.synchronize()
    for b, h in ((0, 1), (3, 2)):
        a = (d["q"][b, h], d["k"][b, h], d["v"][b, h], d["log_alpha_slot"][b, h])
        check(f"o[{b},{h}]", host(o)[b, h], gsa.gsa_fwd(*a), "bf16")
        for kname, t, r in zip(("dq", "dk", "dv", "dla"), g, gsa.gsa_bwd(*a, d["dO"][b, h])):
            check(f"{kname}[{b},{h}]", host(t)[b, h], r, "bf16")


def test_gsa_empty_is_noop(gla):
    z = torch.zeros((1, 2, 0, 64), device=DEV)
    la = torch.zeros((1, 2, 0, 64), device=DEV)
    o = gla.gsa_fwd(z, z, z, la)
    g = gla.gsa_bwd(z, z, z, la, z)
    assert o.shape == (1, 2, 0, 64) and all(t.numel() == 0 for t in g)


def test_gsa_full_size_sampled(gla):
    """B=4, H=4, T=2048, dk=256, dv=512, 64 slots: the forward of one sampled head at full
    length; the backward of one sampled head of a T=512 run of the same shape."""
    cfg = GlaConfig(name="gsa1p3b", dtype="f32", B=4, H=4, T=2048, dk=256, dv=512, chunk=64)
    d = generate_gsa(cfg, 64, with_dO=False)
    x = {n: to_dev(d[n + "_store"], "f32", DEV) for n in ("q", "k", "v", "log_alpha_slot")}
    o = gla.gsa_fwd(x["q"], x["k"], x["v"], x["log_alpha_slot"])
    torch.cuda.synchronize()
    b, h = 2, 3
    ref = gsa.gsa_fwd(d["q"][b, h], d["k"][b, h], d["v"][b, h], d["log_alpha_slot"][b, h])
    check("o[2,3]", host(o)[b, h], ref, "f32")
    cfg2 = cfg.replace(name="gsa1p3b_t512", T=512)
    d2 = generate_gsa(cfg2, 64)
    x2 = _dev(d2)
    g = gla.gsa_bwd(x2["q"], x2["k"], x2["v"], x2["log_alpha_slot"], x2["dO"])
    torch.cuda.synchronize()
    b, h = 1, 0
    a = (d2["q"][b, h], d2["k"][b, h], d2["v"][b, h], d2["log_alpha_slot"][b, h])
    for kname, t, r in zip(("dq", "dk", "dv", "dla"), g, gsa.gsa_bwd(*a, d2["dO"][b, h])):
        check(f"{kname}[1,0]", host(t)[b, h], r, "f32")


def test_gsa_caller_workspace(gla):
    """A caller workspace is checked for size before the call (ValueError when short) and
    a large enough one gives the same output as the library-sized one."""
    cfg = GlaConfig(name="gsaws", dtype="f32", B=1, H=1, T=100, dk=64, dv=64, chunk=64)
    say(f"[gsa] caller workspace {cfg}")
    d = generate_gsa(cfg, 64)
    x = _dev(d)
    desc = gla.make_gsa_desc(1, 1, 100, 64, 64, 64, gla.F32)
    need_f = gla.gsa_workspace_bytes(desc, gla.PASS_FWD)
    need_b = gla.gsa_workspace_bytes(desc, gla.PASS_BWD)
    with pytest.raises(ValueError):
        gla.gsa_fwd(x["q"], x["k"], x["v"], x["log_alpha_slot"],
                    workspace=torch.empty(need_f - 1, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        gla.gsa_bwd(x["q"], x["k"], x["v"], x["log_alpha_slot"], x["dO"],
                    workspace=torch.empty(need_b // 2, dtype=torch.uint8, device=DEV))
    ws = torch.empty(need_b + 4096, dtype=torch.uint8, device=DEV)
    a = gla.gsa_fwd(x["q"], x["k"], x["v"], x["log_alpha_slot"], workspace=ws)
    b = gla.gsa_fwd(x["q"], x["k"], x["v"], x["log_alpha_slot"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
