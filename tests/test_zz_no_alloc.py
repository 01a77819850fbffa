"""The allocation-free forward gla_chunk_fwd_noalloc (scratch from the library's fixed
device array) against gla_chunk_fwd with a caller workspace: the same kernels, so the
outputs must be bit-identical; two calls in a row, the second smaller than the first
(the array keeps the first call's contents).  Called through the C ABI with ctypes.  (That
a problem larger than the array is refused before the device is touched is a host test.)"""
import ctypes

import numpy as np
import pytest

from gla_inputs import GlaConfig, generate
from tests.gpu_util import check, dev_inputs, host, oracle_heads, say

torch = pytest.importorskip("torch")

DEV = "cuda:0"


@pytest.fixture(scope="module")
def nat():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from chunkwise_linear_rnn_amd import _native as m
    m.lib()
    return m


def _P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run_both(nat, cfg, mode, with_S0):
    d = generate(cfg, with_dO=False)
    x = dev_inputs(d, cfg.dtype, DEV, names=("q", "k", "v", "log_alpha"))
    B, H, T, dk, dv = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    desc = nat.make_desc(B, H, T, dk, dv, cfg.chunk, 16,
                         nat.BF16 if cfg.dtype == "bf16" else nat.F32, mode)
    S0 = None
    S0n = None
    if with_S0:
        S0n = np.random.default_rng(3).standard_normal((B, H, dk, dv)).astype(np.float32) * 0.5
        S0 = torch.from_numpy(S0n).to(DEV)
    L = nat.lib()
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    need = nat.workspace_bytes(desc, nat.PASS_FWD)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    o_ref = torch.empty((B, H, T, dv), dtype=dt, device=DEV)
    S_ref = torch.empty((B, H, dk, dv), dtype=torch.float32, device=DEV)
    st = L.gla_chunk_fwd(ctypes.byref(desc), _P(x["q"]), _P(x["k"]), _P(x["v"]),
                         _P(x["log_alpha"]), _P(S0), _P(o_ref), _P(S_ref), _P(ws), need, sp)
    assert st == 0, nat.status_string(st)
    # outputs prefilled with a pattern, so that a missed write shows
    o_na = torch.full((B, H, T, dv), 7.0, dtype=dt, device=DEV)
    S_na = torch.full((B, H, dk, dv), 7.0, dtype=torch.float32, device=DEV)
    st = L.gla_chunk_fwd_noalloc(ctypes.byref(desc), _P(x["q"]), _P(x["k"]), _P(x["v"]),
                                 _P(x["log_alpha"]), _P(S0), _P(o_na), _P(S_na), sp)
    assert st == 0, nat.status_string(st)
    torch.cuda.synchronize()
    return d, S0n, (o_ref, S_ref), (o_na, S_na)


@pytest.mark.gpu
def test_noalloc_matches_workspace_forward(nat):
    # first a large call (fills much of the scratch array), then a smaller one
    cases = [
        (GlaConfig("na_big", "bf16", 4, 4, 2048, 256, 512, 64, seed=8), nat.RECOMPUTE, False),
        (GlaConfig("na_small", "bf16", 1, 2, 300, 128, 128, 64, seed=9), nat.RECOMPUTE, True),
        (GlaConfig("na_small_mat", "f32", 1, 1, 130, 64, 64, 64, seed=10), nat.MATERIALIZED,
         True),
    ]
    for cfg, mode, with_S0 in cases:
        say(f"[noalloc] {cfg} mode={mode} S0={with_S0}")
        d, S0n, (o_ref, S_ref), (o_na, S_na) = _run_both(nat, cfg, mode, with_S0)
        assert torch.equal(o_na, o_ref), "o differs from gla_chunk_fwd"
        assert torch.equal(S_na, S_ref), "S_T differs from gla_chunk_fwd"
        if cfg.B * cfg.H * cfg.T <= 1024:
            heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
            ref = oracle_heads(d, heads, None if S0n is None else S0n.astype(np.float64),
                               bwd=False)
            check("o", np.stack([host(o_na)[b, h] for b, h in heads]), ref["o"], cfg.dtype)
            check("S_T", np.stack([host(S_na)[b, h] for b, h in heads]), ref["S_T"], cfg.dtype)
