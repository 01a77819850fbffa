"""The traced entry points: every stage boundary recorded, or only some (NULL entries in the
event array skip their boundary); the outputs are those of the plain entry points, bit for
bit, and the recorded events bracket positive durations."""
import ctypes

import numpy as np
import pytest

from gla_inputs import GlaConfig, generate
from tests.gpu_util import dev_inputs, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DEV = "cuda:0"


class _Events:
    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def make(self):
        ev = ctypes.c_void_p()
        assert self.h.hipEventCreate(ctypes.byref(ev)) == 0
        self.made.append(ev)
        return ev

    def ms(self, a, b):
        out = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(out), a, b) == 0
        return out.value

    def close(self):
        for ev in self.made:
            self.h.hipEventDestroy(ev)


@pytest.mark.parametrize("which", ["all", "sparse"])
def test_traced_matches_plain(which):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_linear_rnn_amd as gla
    from chunkwise_linear_rnn_amd import _native as nat
    L = nat.lib()
    cfg = GlaConfig("trace", "bf16", 1, 2, 300, 128, 128, 64, seed=21)
    say(f"[trace] {which} {cfg}")
    d = generate(cfg)
    x = dev_inputs(d, "bf16", DEV)
    o_ref, _ = gla.fwd(x["q"], x["k"], x["v"], x["log_alpha"])
    g_ref = gla.bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["dO"])
    desc = nat.make_desc(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk, 16, nat.BF16,
                         nat.RECOMPUTE)
    nfs, nbs = len(nat.trace_stages(desc, nat.PASS_FWD)), len(nat.trace_stages(desc, nat.PASS_BWD))
    E = _Events()
    evf = (ctypes.c_void_p * (nfs + 1))()
    evb = (ctypes.c_void_p * (nbs + 1))()
    if which == "all":
        for j in range(nfs + 1):
            evf[j] = E.make()
        for j in range(nbs + 1):
            evb[j] = E.make()
        timed_f, timed_b = list(range(nfs)), list(range(nbs))
    else:   # the last forward stage and the last backward stage only
        evf[nfs - 1], evf[nfs] = E.make(), E.make()
        evb[nbs - 1], evb[nbs] = E.make(), E.make()
        timed_f, timed_b = [nfs - 1], [nbs - 1]
    o = torch.empty_like(o_ref)
    S_T = torch.empty((cfg.B, cfg.H, cfg.dk, cfg.dv), dtype=torch.float32, device=DEV)
    dq, dk_, dv_, dla = (torch.empty_like(t) for t in (x["q"], x["k"], x["v"], x["log_alpha"]))
    wf, wb = nat.workspace_bytes(desc, nat.PASS_FWD), nat.workspace_bytes(desc, nat.PASS_BWD)
    wsf = torch.empty(wf, dtype=torch.uint8, device=DEV)
    wsb = torch.empty(wb, dtype=torch.uint8, device=DEV)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    assert L.gla_chunk_fwd_traced(ctypes.byref(desc), P(x["q"]), P(x["k"]), P(x["v"]),
                                  P(x["log_alpha"]), None, P(o), P(S_T), P(wsf), wf, sp, evf,
                                  nfs + 1) == 0
    assert L.gla_chunk_bwd_traced(ctypes.byref(desc), P(x["q"]), P(x["k"]), P(x["v"]),
                                  P(x["log_alpha"]), None, P(x["dO"]), None, P(dq), P(dk_),
                                  P(dv_), P(dla), None, P(wsb), wb, sp, evb, nbs + 1) == 0
    # too short an event array is rejected before any launch
    assert L.gla_chunk_fwd_traced(ctypes.byref(desc), P(x["q"]), P(x["k"]), P(x["v"]),
                                  P(x["log_alpha"]), None, P(o), P(S_T), P(wsf), wf, sp, evf,
                                  nfs) != 0
    torch.cuda.synchronize()
    assert np.array_equal(host(o), host(o_ref))
    for got, ref in zip((dq, dk_, dv_, dla), g_ref[:4]):
        assert np.array_equal(host(got), host(ref))
    for j in timed_f:
        assert E.ms(evf[j], evf[j + 1]) > 0.0
    for j in timed_b:
        assert E.ms(evb[j], evb[j + 1]) > 0.0
    E.close()
