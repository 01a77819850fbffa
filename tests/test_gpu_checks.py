"""The gate precondition check (gla_check_gates) and the GLA_DEBUG_CHECKS switch: exact
counts of planted violations (positive, NaN and infinite log_alpha; non-finite gate
logits) for per-key and scalar gates in both types, and, in a child process with the
switch set, a forward refused before any output is touched and an accepted one equal to
the same call without the switch."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from gla_inputs import GlaConfig, generate
from tests.gpu_util import dev_inputs, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def gla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_linear_rnn_amd as m
    m.lib()
    return m


def _plant(t, flat_idx, vals):
    x = t.clone()
    f = x.view(-1)
    for i, v in zip(flat_idx, vals):
        f[i] = v
    return x


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_check_gates_counts(gla, dt):
    cfg = GlaConfig(name="chk", dtype=dt, B=2, H=1, T=300, dk=64, dv=64, chunk=64, seed=4)
    say(f"[checks] {cfg}")
    d = generate(cfg)
    x = dev_inputs(d, dt, DEV, names=("q", "v", "log_alpha", "log_alpha_scalar", "gate_logits"))
    q, v = x["q"], x["v"]
    assert gla.check_gates(q, v, x["log_alpha"]) == 0
    n = x["log_alpha"].numel()
    idx = [0, 5, n // 2, n - 1, 777]
    bad = _plant(x["log_alpha"], idx, [0.5, float("nan"), float("inf"), float("-inf"), 1e-3])
    assert gla.check_gates(q, v, bad) == 5
    # zero is allowed (alpha = 1)
    assert gla.check_gates(q, v, _plant(x["log_alpha"], idx, [0.0] * 5)) == 0
    ns = x["log_alpha_scalar"].numel()
    bad_s = _plant(x["log_alpha_scalar"], [1, ns - 2], [2.0, float("nan")])
    assert gla.check_gates(q, v, x["log_alpha_scalar"]) == 0
    assert gla.check_gates(q, v, bad_s) == 2
    # gate logits: any finite value is allowed, non-finite ones are not
    lg = x["gate_logits"]
    assert gla.check_gates(q, v, lg, gate_tau=16.0) == 0
    assert gla.check_gates(q, v, _plant(lg, idx, [5.0, 3.0, -9.0, 1.0, 2.0]), gate_tau=16.0) == 0
    assert gla.check_gates(q, v, _plant(lg, idx[:3], [float("nan"), float("inf"), 4.0]),
                           gate_tau=16.0) == 2


_CHILD = r"""
import ctypes, json, sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import chunkwise_linear_rnn_amd as g
from gla_inputs import GlaConfig, generate
from tests.gpu_util import dev_inputs
cfg = GlaConfig(name="chk_env", dtype="bf16", B=1, H=2, T=200, dk=64, dv=64, chunk=64, seed=9)
d = generate(cfg)
x = dev_inputs(d, "bf16", "cuda:0")
out = {}
bad = x["log_alpha"].clone()
bad.view(-1)[123] = 0.25
o = torch.full((1, 2, 200, 64), 7.0, dtype=torch.bfloat16, device="cuda:0")
ws = torch.empty(g.workspace_bytes(g.make_desc(1, 2, 200, 64, 64), g.PASS_FWD),
                 dtype=torch.uint8, device="cuda:0")
try:
    g.fwd(x["q"], x["k"], x["v"], bad, workspace=ws)
    out["refused"] = None
except g.GlaError as e:
    out["refused"] = e.code
desc = g.make_desc(1, 2, 200, 64, 64)
st = g.lib().gla_chunk_fwd(ctypes.byref(desc), *(g.ops._ptr(t) for t in
                           (x["q"], x["k"], x["v"], bad)), None, g.ops._ptr(o), None,
                           g.ops._ptr(ws), ws.numel(), g.ops._stream(o.device))
torch.cuda.synchronize()
out["raw_status"] = int(st)
out["o_untouched"] = bool(torch.all(o == 7.0).item())
o2, S2 = g.fwd(x["q"], x["k"], x["v"], x["log_alpha"])
torch.cuda.synchronize()
np.save(sys.argv[2], o2.float().cpu().numpy())
print(json.dumps(out))
"""


def test_debug_checks_switch(gla, tmp_path):
    cfg = GlaConfig(name="chk_env", dtype="bf16", B=1, H=2, T=200, dk=64, dv=64, chunk=64, seed=9)
    d = generate(cfg)
    x = dev_inputs(d, "bf16", DEV)
    o_ref, _ = gla.fwd(x["q"], x["k"], x["v"], x["log_alpha"])
    torch.cuda.synchronize()
    say("[checks] child process with GLA_DEBUG_CHECKS=1")
    env = dict(os.environ, GLA_DEBUG_CHECKS="1")
    path = str(tmp_path / "o.npy")
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT, path], env=env, capture_output=True,
                       text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["refused"] == 1 and out["raw_status"] == 1 and out["o_untouched"], out
    assert np.array_equal(np.load(path), o_ref.float().cpu().numpy())
