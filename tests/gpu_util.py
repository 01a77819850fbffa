"""Helpers for the GPU parity tests: move seeded inputs to the device, run the fp64
oracle on sampled (batch, head) pairs, compare with the stated tolerances."""
from __future__ import annotations

import sys

import numpy as np

from oracle import recurrence_fwd, recurrence_bwd
from oracle.compare import max_rel, normwise

# Accuracy bars: fp32 inputs max relative error <= 1e-4; bf16 inputs max relative error
# <= 2e-2 and normwise <= 5e-3 (per output tensor, against the fp64 oracle).
TOL = {"f32": {"max_rel": 1e-4, "normwise": 1e-4}, "bf16": {"max_rel": 2e-2, "normwise": 5e-3}}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arr_store, dtype, device):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr_store)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(arr_store).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def dev_inputs(d, dtype, device, names=("q", "k", "v", "log_alpha", "dO")):
    return {n: to_dev(d[n + "_store"], dtype, device) for n in names if n + "_store" in d}


def host(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def check(name, got, ref, dtype, extra=None):
    tol = TOL[dtype]
    mr, nw = max_rel(got, ref), normwise(got, ref)
    say(f"    {name:12s} max_rel={mr:.3e} normwise={nw:.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert mr <= tol["max_rel"], f"{name}: max_rel {mr:.3e} > {tol['max_rel']}"
    assert nw <= tol["normwise"], f"{name}: normwise {nw:.3e} > {tol['normwise']}"
    return mr, nw


def oracle_heads(d, heads, S0=None, dS_T=None, bwd=True):
    """Oracle outputs for the listed (b, h) pairs, each [len(heads), T, d]."""
    out = {k: [] for k in ("o", "S_T", "dq", "dk", "dv", "dla", "dS0")}
    for b, h in heads:
        sl = (b, h)
        s0 = None if S0 is None else S0[sl]
        dst = None if dS_T is None else dS_T[sl]
        o, ST = recurrence_fwd(d["q"][sl], d["k"][sl], d["v"][sl], d["log_alpha"][sl], s0)
        out["o"].append(o)
        out["S_T"].append(ST)
        if bwd:
            g = recurrence_bwd(d["q"][sl], d["k"][sl], d["v"][sl], d["log_alpha"][sl],
                               d["dO"][sl], s0, dst)
            for kname, val in zip(("dq", "dk", "dv", "dla", "dS0"), g):
                out[kname].append(val)
    return {k: np.stack(v) for k, v in out.items() if v}


def pick(arr, heads):
    return np.stack([arr[b, h] for b, h in heads])


def _oracle_one(args):
    """One (batch, head) of the oracle (runs in a worker process)."""
    q, k, v, la, dO, s0, dst, bwd = args
    o, ST = recurrence_fwd(q, k, v, la, s0)
    out = {"o": o, "S_T": ST}
    if bwd:
        g = recurrence_bwd(q, k, v, la, dO, s0, dst)
        out.update(zip(("dq", "dk", "dv", "dla", "dS0"), g))
    return out


def pool_workers(n_jobs):
    """Worker processes for the oracle: the host's cores available to this process,
    at most 16 (a one-GPU share of the host) and at most one per job."""
    import os
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return max(1, min(16, cores, n_jobs))


def oracle_heads_pool(d, heads, S0=None, dS_T=None, bwd=True):
    """oracle_heads for many (b, h) pairs at once: one process per head (spawned, BLAS
    single-threaded), the same fp64 oracle functions."""
    import multiprocessing as mp
    import os
    jobs = []
    for b, h in heads:
        jobs.append((d["q"][b, h], d["k"][b, h], d["v"][b, h], d["log_alpha"][b, h],
                     d["dO"][b, h] if bwd else None,
                     None if S0 is None else S0[b, h], None if dS_T is None else dS_T[b, h],
                     bwd))
    keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {key: os.environ.get(key) for key in keys}
    for key in keys:
        os.environ[key] = "1"
    try:
        with mp.get_context("spawn").Pool(pool_workers(len(jobs))) as pool:
            res = pool.map(_oracle_one, jobs, chunksize=1)
    finally:
        for key, val in saved.items():
            if val is None:
                os.environ.pop(key, None)
            else:
                os.environ[key] = val
    return {key: np.stack([r[key] for r in res]) for key in res[0]}


def check_heads(name, got, ref, heads, dtype):
    """check() on every (b, h) pair of `heads` separately (got: [B, H, ...] host array,
    ref: [len(heads), ...]), then on all of them together; returns the worst per-head
    (max_rel, normwise)."""
    tol = TOL[dtype]
    worst_mr = worst_nw = 0.0
    for j, (b, h) in enumerate(heads):
        g, r = got[b, h], ref[j]
        mr, nw = max_rel(g, r), normwise(g, r)
        assert np.all(np.isfinite(g)), f"{name} head {(b, h)}: non-finite values"
        assert mr <= tol["max_rel"], f"{name} head {(b, h)}: max_rel {mr:.3e} > {tol['max_rel']}"
        assert nw <= tol["normwise"], f"{name} head {(b, h)}: normwise {nw:.3e} > {tol['normwise']}"
        worst_mr, worst_nw = max(worst_mr, mr), max(worst_nw, nw)
    say(f"    {name:12s} {len(heads)} heads: worst max_rel={worst_mr:.3e} "
        f"worst normwise={worst_nw:.3e}")
    check(name, pick(got, heads), ref, dtype)
    return worst_mr, worst_nw
