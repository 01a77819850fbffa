#!/usr/bin/env python3
"""Throughput of the chunkwise GLA layer, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gla1p3b_t2k]

A step is one training pair, gla_chunk_fwd_save plus gla_chunk_bwd_saved (the forward
keeps the intra-chunk operands for the backward, which then skips its intra-chunk kernel),
over the whole batch of seeded synthetic inputs (already resident in device memory), with every output and workspace
preallocated.  K steps are timed between two device synchronisations; every kernel
launch is also bracketed by HIP events (the traced entry points of the C ABI, recorded
on the stream the kernels run on) to get each stage's average duration.  One JSON line
goes to stdout; a per-stage table goes to stderr.

The roofline object describes the stage with the largest time per step, against the
MI355X peak for its bound (HBM 8 TB/s, or dense bf16 MFMA 2.5 PFLOP/s); its `achieved`
uses the algorithmic bytes or flops per launch from stage_work() below.  `traffic`
is the measured HBM bytes per launch of that stage from the committed rocprofv3 counter
summary, or null when no summary matches the current kernel source.

`recompute_pair_step` times the other pair, gla_chunk_fwd plus gla_chunk_bwd (the backward
rebuilds the intra-chunk operands; nothing is kept between the passes), back to back like
`warm_cache`; `--pair recompute` makes it the timed step instead.

`decode_step` times the recurrent entry point (one token per sequence, float32 state
read and written in place) at the workload's head shape for a small and a serving-size
batch, against the HBM roofline.

`gate_logits_step` times the same step fed gate logits (the gate front-end: log_alpha =
logsigmoid(x)/16 formed inside the kernels, the gradient returned for x), and
`scalar_gate_step` fed scalar gates (one per token and head, [B, H, T]; the gradient is
summed over the key dimension).

`gsa_step` and `gsa_step_bf16` time Gated Slot Attention (fwd + bwd, float32 and bf16,
--gsa-slots memory slots, default 64) at the workload's B, H, T, dk, dv.

Every timed step runs after an untimed cache flush (a 512 MiB device write, then a
512 MiB read that evicts the write's own dirty lines), with HIP events around the step
only: the headline `value` is the cache-flushed rate, the inputs resident in HBM but not
in L2 or the 256 MiB Infinity Cache, and no write-backs of foreign data pending.
`warm_cache` repeats the steps back to back without the flush (inputs and workspaces
partly served from the Infinity Cache), for context.

The CPU baseline times the fp64 oracle (step recurrence, then direct backward, each
timed separately) on a bounded sample of the same workload with a process pool on the
host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import statistics
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # bytes/s
PEAK_BF16 = 2.5e15         # dense bf16 MFMA flop/s
PEAK_F32 = 157.3e12        # fp32 (MFMA / packed vector) flop/s
METRIC = "GLA fwd+bwd tokens/s at 1.3B shape T=2K, 1 GPU; % of bf16 MFMA peak"
HEADLINE_WORKLOAD = "gla1p3b_t2k"


def metric_name(cfg, fwd_only):
    """The headline metric for the 1.3B T=2K shape; any other workload is named by its
    own shape, so that a line never claims a shape it did not run."""
    passes = "fwd" if fwd_only else "fwd+bwd"
    if cfg.name == HEADLINE_WORKLOAD and not fwd_only:
        return METRIC
    return (f"GLA {passes} tokens/s, {cfg.name} (B={cfg.B} H={cfg.H} T={cfg.T} "
            f"dk={cfg.dk} dv={cfg.dv} C={cfg.chunk}), 1 GPU")



def stage_work(stage, pass_, mode, B, H, T, dk, dv, C, e, save=False):
    """(algorithmic HBM bytes, algorithmic flops) of one launch of `stage`.

    Per token and head: each tensor the stage must read or write once, in its storage
    type; flops count a multiply-add as 2 and the causal intra-chunk products at half
    the chunk (C/2 average partners).  `save`: the forward of the training pair, whose
    intra-chunk kernel also writes the backward's operands and whose Kh^T is stored as
    fp32 (with bf16 inputs: a bf16 high part and remainder, 4 bytes an element, of which
    the forward's later kernels read the high part alone)."""
    BH, N = B * H, (T + C - 1) // C
    tok = BH * T
    tokp = BH * N * C                      # padded rows of per-chunk operands
    st = BH * N * dk * dv * e              # one materialized state tensor
    if stage == "intra":
        if pass_ == "fwd" and save:
            # reads log_alpha, q, k; writes A, Qh and Kh (storage type), Qh^T and Kh^T
            # (fp32), e^gamma
            byt = (3 * tok * dk * e + 2 * tokp * dk * e + 2 * tokp * dk * 4
                   + BH * N * C * C * e + BH * N * dk * 4)
        elif pass_ == "fwd":
            byt = 3 * tok * dk * e + 2 * tokp * dk * e + BH * N * C * C * e + BH * N * dk * 4
        else:   # reads log_alpha, q, k; writes A, Qh^T, Kh^T (fp32), Kh, e^gamma (the
            # chunk kernel rebuilds g itself)
            byt = (3 * tok * dk * e + BH * N * C * C * e + 2 * tokp * dk * 4 + tokp * dk * e
                   + BH * N * dk * 4)
        return byt, tok * C * dk
    if stage in ("state_scan_fwd", "state_scan_rev", "state_scans"):
        # one scan: reads Kh^T and Qh^T (fp32 as bf16 pairs), v and dO; writes the states
        # and the cross-term tiles.  state_scans is both scans in one launch.
        byt = 2 * tokp * dk * 4 + 2 * tok * dv * e + st + BH * N * (dv // 64) * dk * 4
        n = 2 if stage == "state_scans" else 1
        return n * byt, n * tok * 4 * dk * dv
    if stage == "state_scan":
        return tokp * dk * e + tok * dv * e + st + BH * dk * dv * 4, tok * 2 * dk * dv
    if stage == "output":
        return tokp * dk * e + BH * N * C * C * e + st + 2 * tok * dv * e, tok * (2 * dk * dv + C * dv)
    if stage == "seg_state":
        # the states at the segment starts: Kh^T and v of every segment but the last, the
        # end state of each scanned segment, and (more than two segments) their chaining
        P = fused_segments(e, C, N, BH, dv)
        ns = (P - 1) * N // P
        h = BH * ns * C
        st4 = BH * dk * dv * 4
        byt = h * dk * e + h * dv * e + BH * ns * dk * 4 + (P - 1) * st4
        if P > 2:
            byt += 2 * (P - 2) * st4
        return byt, h * 2 * dk * dv
    if stage == "fwd_fused":
        byt = 2 * tokp * dk * e + BH * N * C * C * e + 2 * tok * dv * e + BH * dk * dv * 4
        return byt, tok * (4 * dk * dv + C * dv)
    if stage == "bwd_dqk_dv":
        # dq/dk part: reads q, k, v, dO, log_alpha, S, dS, chunk totals; writes dq, dk, dla
        byt = (tok * (2 * dk * e + 2 * dv * e + dk * e) + 2 * st + BH * N * dk * 4
               + tok * 3 * dk * e)
        fl = tok * (4 * dk * dv + C * dv + 2 * C * dk)
        # dv part: reads Kh, A (dS and dO are the dq/dk part's, read once by the launch);
        # writes dv
        byt += tokp * dk * e + BH * N * C * C * e + tok * dv * e
        fl += tok * (2 * dk * dv + C * dv)
        return byt, fl
    if stage == "gate_tot":
        return 2 * BH * N * (dv // 64) * dk * 4 + BH * N * dk * 4, 0
    if stage == "state_dot":
        return 2 * BH * dk * dv * 4, 2 * BH * dk * dv
    return 0, 0


def fused_segments(e, C, N, BH, dv):
    """Sequence segments of the non-materialized forward, as the library picks them: about
    256 workgroups (one per CU) for small B*H*dv/64, at most 8, at least two chunks each;
    none for fp32 or fewer than 4 chunks."""
    if e == 4 or N < 4:
        return 1
    tiles = BH * (dv // 64)
    P = 2 if tiles >= 128 else 256 // tiles
    return max(2, min(P, 8, N // 2))


def path_flops(B, H, T, dk, dv, C, fwd_only=False):
    """Algorithmic flops of one forward + backward, or of the forward alone (causal intra
    counted at C/2)."""
    tok = B * H * T
    fwd = tok * (4 * dk * dv + C * (dk + dv))
    return fwd if fwd_only else fwd + tok * (8 * dk * dv + C * (3 * dk + 2 * dv))


# ---------------------------------------------------------------------------------
# HIP events through the runtime the library uses
# ---------------------------------------------------------------------------------
class HipEvents:
    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, ev, stream):
        if self.h.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def create(self, n):
        arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.h.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = ev
        return arr

    def elapsed_ms(self, a, b):
        out = ctypes.c_float()
        err = self.h.hipEventElapsedTime(ctypes.byref(out), a, b)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return float(out.value)

    def destroy(self, arr):
        for ev in arr:
            self.h.hipEventDestroy(ev)


# ---------------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------------
def _oracle_warm(_):
    import numpy  # noqa: F401
    import oracle  # noqa: F401
    return 0


def _oracle_fwd(args):
    q, k, v, la, dO = args
    from oracle import recurrence_fwd
    recurrence_fwd(q, k, v, la)


def _oracle_bwd(args):
    q, k, v, la, dO = args
    from oracle import recurrence_bwd
    recurrence_bwd(q, k, v, la, dO)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(d, cfg, T_sample):
    import multiprocessing as mp
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    workers = max(1, min(16, cores, cfg.B * cfg.H))
    heads = [(i // cfg.H, i % cfg.H) for i in range(workers)]
    jobs = [tuple(d[n][b, h, :T_sample].copy() for n in ("q", "k", "v", "log_alpha", "dO"))
            for b, h in heads]
    env_before = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                 "MKL_NUM_THREADS")}
    for k in env_before:
        os.environ[k] = "1"
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_warm, range(workers))      # process start-up is not timed
        t0 = time.perf_counter()
        pool.map(_oracle_fwd, jobs, chunksize=1)
        t1 = time.perf_counter()
        pool.map(_oracle_bwd, jobs, chunksize=1)
        t2 = time.perf_counter()
    wall_f, wall_b = t1 - t0, t2 - t1
    wall = wall_f + wall_b
    for k, val in env_before.items():
        if val is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = val
    tokens = workers * T_sample / cfg.H     # head-tokens -> tokens (each token has H heads)
    # cores: the worker processes (one thread each) that ran the oracle; host_cores: the
    # cores available to this process on the host
    return {"value": tokens / wall, "unit": "tokens/s", "cores": workers,
            "host_cores": cores, "workers": workers, "kind": "oracle",
            "sample": (f"fp64 step recurrence + direct backward, {workers} (batch, head) pairs x "
                       f"first {T_sample} tokens of {cfg.name}, one process per head, "
                       f"{wall:.2f} s wall (fwd {wall_f:.2f} s, bwd {wall_b:.2f} s)"),
            "fwd_s": wall_f, "bwd_s": wall_b, "cpu_model": _cpu_model()}


BWD_SHARED = ("bwd_dqk_dv", "state_scans", "state_dot", "gate_tot")


def counter_traffic(stage, workload, kind="recompute"):
    """HBM bytes per launch from a committed counter summary that matches the current
    kernel source, else None.  `kind`: "recompute" (the training pair in recompute state
    mode, the summaries without suffix), "materialized" or "recompute_pair", whose
    summaries carry that suffix; the backward's scans and its dq/dk/dv and gate kernels
    are the same launches in all three, so those fall back to the summary without
    suffix."""
    path = os.path.join(ROOT, "profiles", f"counters_{stage}_{workload}.json")
    if kind != "recompute":
        mpath = os.path.join(ROOT, "profiles", f"counters_{stage}_{workload}_{kind}.json")
        if os.path.exists(mpath):
            path = mpath
        elif stage not in BWD_SHARED:
            return None
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    from chunkwise_linear_rnn_amd.profiling import STAGE_SOURCE, source_digest
    if stage not in STAGE_SOURCE or rec.get("source_sha256") != source_digest(stage, ROOT):
        return None
    return rec.get("traffic_bytes_per_launch")


def counter_mfma(workload, kind):
    """Matrix-unit figures per stage from the committed `rocprofv3 --pmc
    SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE` summary of this
    workload and kind (as counter_traffic): {stage: {mfma_busy_frac, bf16_peak_frac, ...}}
    for the stages whose kernel source still matches the summary's hash; {} when there is
    none."""
    suffix = "" if kind == "recompute" else "_" + kind
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}{suffix}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as fh:
        rec = json.load(fh)
    from chunkwise_linear_rnn_amd.profiling import source_digest
    out = {}
    for kr in rec.get("kernels", []):
        for st in kr.get("stages", []):
            if rec.get("source_sha256", {}).get(st) != source_digest(st, ROOT):
                continue
            out[st] = {"mfma_busy_frac": kr["mfma_busy_frac"],
                       "bf16_peak_frac": kr["bf16_peak_frac"],
                       "bf16_gflop_per_launch": kr["bf16_gflop_per_launch"],
                       "summary": os.path.relpath(path, ROOT)}
    return out


def gsa_measure(L, nat, hip, dev, sp, cfg, slots, steps, dtype="f32"):
    """Gated Slot Attention fwd + bwd (gla_gsa_fwd, gla_gsa_bwd; float32 or bf16) on the
    workload's B, H, T, dk, dv with `slots` memory slots: ms per step from HIP events
    around `steps` back-to-back steps after 2 warm-up steps.  Inputs:
    gla_inputs.generate_gsa."""
    import numpy as np
    import torch
    from gla_inputs import generate_gsa
    cd = cfg.replace(dtype=dtype)
    d = generate_gsa(cd, slots)

    def up(n):
        a = np.ascontiguousarray(d[n + "_store"])
        if dtype == "f32":
            return torch.from_numpy(a).to(dev)
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    t = {n: up(n) for n in ("q", "k", "v", "dO", "log_alpha_slot")}
    desc = nat.make_gsa_desc(cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, slots,
                             nat.F32 if dtype == "f32" else nat.BF16)
    o = torch.empty_like(t["v"])
    grads = [torch.empty_like(t[n]) for n in ("q", "k", "v", "log_alpha_slot")]
    need_f = nat.gsa_workspace_bytes(desc, nat.PASS_FWD)
    need_b = nat.gsa_workspace_bytes(desc, nat.PASS_BWD)
    ws = torch.empty(max(need_f, need_b), dtype=torch.uint8, device=dev)
    P = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731

    def step():
        for st in (L.gla_gsa_fwd(ctypes.byref(desc), P(t["q"]), P(t["k"]), P(t["v"]),
                                 P(t["log_alpha_slot"]), P(o), P(ws), need_f, sp),
                   L.gla_gsa_bwd(ctypes.byref(desc), P(t["q"]), P(t["k"]), P(t["v"]),
                                 P(t["log_alpha_slot"]), P(t["dO"]), *(P(g) for g in grads),
                                 P(ws), need_b, sp)):
            if st:
                raise nat.GlaError(st, "gla_gsa_fwd/bwd")
    for _ in range(2):
        step()
    evs = hip.create(2)
    hip.record(evs[0], sp)
    for _ in range(steps):
        step()
    hip.record(evs[1], sp)
    torch.cuda.synchronize()
    ms = hip.elapsed_ms(evs[0], evs[1]) / steps
    hip.destroy(evs)
    return {"ms_per_step": ms, "value": cfg.B * cfg.T / (ms * 1e-3), "unit": "tokens/s",
            "slots": slots, "dtype": dtype, "steps": steps}


def decode_measure(L, nat, hip, dev, sp, H, dk, dv, batches=(4, 64), calls=200):
    """One-token recurrent steps (gla_decode, T = 1, bf16, float32 state in place) at a few
    batch sizes: microseconds per step from HIP events around `calls` back-to-back steps;
    the algorithmic bytes are the state read and written plus the token's q, k, v,
    log_alpha and o."""
    import torch
    out = []
    for B in batches:
        g = torch.Generator(device="cpu").manual_seed(B)
        mk = lambda *s: (torch.randn(*s, generator=g) * 0.1).to(torch.bfloat16).to(dev)  # noqa: E731
        q, k, la = mk(B, H, 1, dk), mk(B, H, 1, dk), -mk(B, H, 1, dk).abs()
        v = mk(B, H, 1, dv)
        S = torch.zeros((B, H, dk, dv), dtype=torch.float32, device=dev)
        o = torch.empty((B, H, 1, dv), dtype=torch.bfloat16, device=dev)
        desc = nat.make_desc(B, H, 1, dk, dv, 64, 16, nat.BF16, nat.RECOMPUTE)
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        args = (ctypes.byref(desc), P(q), P(k), P(v), P(la), P(S), P(o), sp)
        for _ in range(20):
            if L.gla_decode(*args):
                raise nat.GlaError(L.gla_decode(*args), "gla_decode")
        evs = hip.create(2)
        hip.record(evs[0], sp)
        for _ in range(calls):
            L.gla_decode(*args)
        hip.record(evs[1], sp)
        torch.cuda.synchronize()
        us = hip.elapsed_ms(evs[0], evs[1]) * 1e3 / calls
        hip.destroy(evs)
        byt = 2 * B * H * dk * dv * 4 + B * H * (3 * dk + 2 * dv) * 2
        out.append({"B": B, "H": H, "dk": dk, "dv": dv, "us_per_step": us,
                    "tokens_per_s": B / (us * 1e-6), "algorithmic_bytes": byt,
                    "achieved_GBps": byt / (us * 1e-6) / 1e9,
                    "hbm_frac": byt / (us * 1e-6) / PEAK_HBM})
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE_WORKLOAD)
    ap.add_argument("--state-mode", default="recompute", choices=["recompute", "materialized"])
    ap.add_argument("--pair", default="train", choices=["train", "recompute"],
                    help="the timed step: the training pair (the forward keeps the "
                         "intra-chunk operands for the backward) or the recompute pair; the "
                         "materialized state mode and forward-only workloads time the latter")
    ap.add_argument("--scalar-gates", action="store_true",
                    help="time the step with scalar gates (one per token and head, [B, H, T]) "
                         "as the main measurement, with its per-stage table")
    ap.add_argument("--diag", default="f32", choices=["f32", "bf16"],
                    help="arithmetic of the diagonal intra-chunk sub-blocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the side measurements: decode step, gate-logit and scalar-gate "
                         "steps, Gated Slot Attention step")
    ap.add_argument("--gsa-slots", type=int, default=64,
                    help="memory slots of the Gated Slot Attention step")
    ap.add_argument("--gsa-only", action="store_true",
                    help="time only the Gated Slot Attention step and print its JSON (for "
                         "profiling its kernels on their own)")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens per (batch, head) in the oracle sample")
    ap.add_argument("--no-flush", action="store_true",
                    help="time the steps back to back without the cache-evicting write "
                         "(then `value` is the warm-cache rate)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (sharding is a "
              "design note only); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import chunkwise_linear_rnn_amd as gla
    from chunkwise_linear_rnn_amd import _native as nat
    from gla_inputs import CONFIGS, generate

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.gsa_only:
        L = nat.lib()
        sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        hip_ = HipEvents()
        rec = gsa_measure(L, nat, hip_, dev, sp, cfg, args.gsa_slots, args.steps)
        rec.update({"metric": "Gated Slot Attention fwd+bwd tokens/s", "n_gpus": 1,
                    "config": {"workload": cfg.name + f"_gsa{args.gsa_slots}", "B": cfg.B,
                               "H": cfg.H, "T": cfg.T, "dk": cfg.dk, "dv": cfg.dv}})
        rec["bf16"] = gsa_measure(L, nat, hip_, dev, sp, cfg, args.gsa_slots, args.steps, "bf16")
        print(json.dumps(rec), flush=True)
        return
    print(f"[bench] generating {cfg}", file=sys.stderr, flush=True)
    d = generate(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def up(name):
        a = d[name + "_store"]
        if cfg.dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, k, v, la, dO = (up(n) for n in ("q", "k", "v", "log_alpha", "dO"))
    if args.scalar_gates:
        la = up("log_alpha_scalar")
    B, H, T, dk, dv, C = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.chunk
    mode = nat.RECOMPUTE if args.state_mode == "recompute" else nat.MATERIALIZED
    desc = nat.make_desc(B, H, T, dk, dv, C, cfg.subchunk, nat.BF16 if cfg.dtype == "bf16" else nat.F32, mode,
                         gate_shape=nat.GATE_SCALAR if args.scalar_gates else nat.GATE_PER_KEY,
                         diag=nat.DIAG_BF16 if args.diag == "bf16" else nat.DIAG_F32)
    o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    dq, dk_, dv_, dla = (torch.empty_like(x) for x in (q, k, v, la))
    # a forward-only workload (the long sequence with state carry) times gla_chunk_fwd alone
    fwd_only = not cfg.bwd
    train = args.pair == "train" and mode == nat.RECOMPUTE and not fwd_only
    pass_f, pass_b = (nat.PASS_FWD_SAVE, nat.PASS_BWD_SAVED) if train else (nat.PASS_FWD, nat.PASS_BWD)
    wsf_n = nat.workspace_bytes(desc, pass_f)
    wsb_n = nat.workspace_bytes(desc, pass_b)
    wsf = torch.empty(max(1, wsf_n), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, wsb_n), dtype=torch.uint8, device=dev)
    sv_n = nat.saved_bytes(desc) if train else 0
    saved = torch.empty(max(1, sv_n), dtype=torch.uint8, device=dev)
    fwd_stages = nat.trace_stages(desc, pass_f)
    bwd_stages = [] if fwd_only else nat.trace_stages(desc, pass_b, False)
    nf, nb = len(fwd_stages) + 1, len(bwd_stages) + 1
    L = nat.lib()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    hip = HipEvents()
    # Events at every stage boundary cost ~3-4 us each (they serialize the launches around
    # them), so they are recorded in full only in the warm-up (to find the longest stage)
    # and in a profiling pass after the timed region; the timed steps record just the two
    # events around the longest stage (NULL entries skip their boundary).
    evf = [hip.create(nf) for _ in range(args.warmup)]
    evb = [hip.create(nb) for _ in range(args.warmup)]

    def step(ef, eb):
        n_ef, n_eb = (nf if ef is not None else 0), (nb if eb is not None else 0)
        if train:
            st = L.gla_chunk_fwd_save_traced(ctypes.byref(desc), P(q), P(k), P(v), P(la), None,
                                             P(o), P(S_T), P(saved), sv_n, P(wsf), wsf_n, sp,
                                             ef, n_ef)
        else:
            st = L.gla_chunk_fwd_traced(ctypes.byref(desc), P(q), P(k), P(v), P(la), None, P(o),
                                        P(S_T), P(wsf), wsf_n, sp, ef, n_ef)
        if st:
            raise nat.GlaError(st, "forward (traced)")
        if fwd_only:
            return
        if train:
            st = L.gla_chunk_bwd_saved_traced(ctypes.byref(desc), P(q), P(k), P(v), P(la), None,
                                              P(dO), None, P(dq), P(dk_), P(dv_), P(dla), None,
                                              P(saved), sv_n, P(wsb), wsb_n, sp, eb, n_eb)
        else:
            st = L.gla_chunk_bwd_traced(ctypes.byref(desc), P(q), P(k), P(v), P(la), None, P(dO),
                                        None, P(dq), P(dk_), P(dv_), P(dla), None, P(wsb), wsb_n,
                                        sp, eb, n_eb)
        if st:
            raise nat.GlaError(st, "backward (traced)")

    def stage_means(evs_f, evs_b, n_steps, agg=statistics.fmean):
        acc = {}
        for j in range(n_steps):
            for names, evs, tag in ((fwd_stages, evs_f[j], "fwd"), (bwd_stages, evs_b[j], "bwd")):
                for s_i, name in enumerate(names):
                    acc.setdefault((tag, name), []).append(hip.elapsed_ms(evs[s_i], evs[s_i + 1]))
        return {key: agg(ms) for key, ms in acc.items()}

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for j in range(args.warmup):
        step(evf[j], evb[j])
    torch.cuda.synchronize()
    # per-stage medians: the first steps carry one-off costs (first launches, cold caches)
    warm = stage_means(evf, evb, args.warmup, statistics.median) if args.warmup > 0 else {}
    # the stage the roofline describes: the longest in the warm-up (a stage with no launch
    # for this shape reads ~0)
    dom_key = max(warm, key=warm.get) if warm else ("bwd", bwd_stages[-1])
    dom_pass, dom_i = dom_key[0], (fwd_stages if dom_key[0] == "fwd" else bwd_stages).index(dom_key[1])
    ev_dom = [hip.create(2) for _ in range(args.steps)]
    sparse = []
    for j in range(args.steps):
        arr = (ctypes.c_void_p * (nf if dom_pass == "fwd" else nb))()
        arr[dom_i], arr[dom_i + 1] = ev_dom[j][0], ev_dom[j][1]
        sparse.append(arr)

    # The timed steps: each after an untimed flush, HIP events around the step itself, and
    # the two events around the longest stage.  The flush writes 512 MiB and then reads
    # another 512 MiB: the write evicts the previous step's data from L2 and the 256 MiB
    # Infinity Cache, and the read evicts the write's own dirty lines, so that the timed
    # step starts with none of its data cached and no foreign write-backs pending (a
    # write alone left ~256 MiB of dirty lines that the timed step then paid to write back).
    flush = not args.no_flush
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if flush else None
    scratch_rd = (torch.empty(128 << 20, dtype=torch.float32, device=dev).fill_(1.0)
                  if flush else None)
    ev_step = [hip.create(2) for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps{' (cache flushed before each)' if flush else ''}",
          file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        if flush:
            scratch.fill_(j & 0xFF)
            scratch_rd.sum()
        hip.record(ev_step[j][0], sp)
        if dom_pass == "fwd":
            step(sparse[j], None)
        else:
            step(None, sparse[j])
        hip.record(ev_step[j][1], sp)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = sum(hip.elapsed_ms(e0, e1) for e0, e1 in ev_step) / args.steps
    dom_ms = sum(hip.elapsed_ms(ev_dom[j][0], ev_dom[j][1]) for j in range(args.steps)) / args.steps
    del scratch, scratch_rd

    # The same steps back to back without the flush (warm Infinity Cache), for context.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        step(None, None)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    warm_rec = {"ms_per_step": warm_ms, "value": B * T / (warm_ms * 1e-3), "steps": args.steps}

    # per-stage means from a profiling pass of the same steps with every boundary recorded
    n_prof = args.steps
    pf = [hip.create(nf) for _ in range(n_prof)]
    pb = [hip.create(nb) for _ in range(n_prof)]
    t0 = time.perf_counter()
    for j in range(n_prof):
        step(pf[j], pb[j])
    torch.cuda.synchronize()
    traced_ms = (time.perf_counter() - t0) * 1e3 / n_prof
    stages = stage_means(pf, pb, n_prof)
    gpu_ms_from_events = sum(stages.values())
    evf += pf
    evb += pb

    # The same steps with other gate inputs: gate logits (log_alpha = logsigmoid(x)/16
    # formed in the kernels, the gradient returned for x), and scalar gates (one per token,
    # [B, H, T], gradient summed over the key dimension).
    def time_variant(desc_v, gate_t, dla_t, what, train_v=train):
        pf_, pb_ = (nat.PASS_FWD_SAVE, nat.PASS_BWD_SAVED) if train_v else (nat.PASS_FWD, nat.PASS_BWD)
        ws_f = torch.empty(max(1, nat.workspace_bytes(desc_v, pf_)), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(max(1, nat.workspace_bytes(desc_v, pb_)), dtype=torch.uint8, device=dev)
        sv = torch.empty(max(1, nat.saved_bytes(desc_v) if train_v else 1), dtype=torch.uint8,
                         device=dev)
        evs = hip.create(2)

        def step_v():
            if train_v:
                calls = (L.gla_chunk_fwd_save(ctypes.byref(desc_v), P(q), P(k), P(v), P(gate_t),
                                              None, P(o), P(S_T), P(sv), sv.numel(), P(ws_f),
                                              ws_f.numel(), sp),
                         lambda: L.gla_chunk_bwd_saved(ctypes.byref(desc_v), P(q), P(k), P(v),
                                                       P(gate_t), None, P(dO), None, P(dq),
                                                       P(dk_), P(dv_), P(dla_t), None, P(sv),
                                                       sv.numel(), P(ws_b), ws_b.numel(), sp))
            else:
                calls = (L.gla_chunk_fwd(ctypes.byref(desc_v), P(q), P(k), P(v), P(gate_t), None,
                                         P(o), P(S_T), P(ws_f), ws_f.numel(), sp),
                         lambda: L.gla_chunk_bwd(ctypes.byref(desc_v), P(q), P(k), P(v),
                                                 P(gate_t), None, P(dO), None, P(dq), P(dk_),
                                                 P(dv_), P(dla_t), None, P(ws_b), ws_b.numel(),
                                                 sp))
            if calls[0]:
                raise nat.GlaError(calls[0], f"forward with {what}")
            st = calls[1]()
            if st:
                raise nat.GlaError(st, f"backward with {what}")
        for _ in range(3):
            step_v()
        n_v = max(5, args.steps // 2)
        hip.record(evs[0], sp)
        for _ in range(n_v):
            step_v()
        hip.record(evs[1], sp)
        torch.cuda.synchronize()
        vms = hip.elapsed_ms(evs[0], evs[1]) / n_v
        hip.destroy(evs)
        del ws_f, ws_b, sv
        return {"ms_per_step": vms, "value": B * T / (vms * 1e-3), "steps": n_v}

    gate_fe = scalar_fe = other_pair = None
    if not args.no_decode and not fwd_only:
        if mode == nat.RECOMPUTE:
            other_pair = time_variant(desc, la, dla, "the other pair", not train)
            other_pair["pair"] = "recompute" if train else "train"
        dt_code = nat.BF16 if cfg.dtype == "bf16" else nat.F32
        desc_g = nat.make_desc(B, H, T, dk, dv, C, cfg.subchunk, dt_code, mode, nat.GATE_LOGITS,
                               16.0)
        gate_fe = time_variant(desc_g, up("gate_logits"), dla, "gate logits")
        gate_fe["gate_tau"] = 16.0
        desc_s = nat.make_desc(B, H, T, dk, dv, C, cfg.subchunk, dt_code, mode,
                               gate_shape=nat.GATE_SCALAR)
        la_s = up("log_alpha_scalar")
        dla_s = torch.empty_like(la_s)
        scalar_fe = time_variant(desc_s, la_s, dla_s, "scalar gates")

    # Gated Slot Attention (float32 and bf16) at the workload's head shape: fwd + bwd steps
    gsa_step = gsa_step_h = None
    if not args.no_decode and not fwd_only:
        gsa_step = gsa_measure(L, nat, hip, dev, sp, cfg, args.gsa_slots, max(5, args.steps // 5))
        gsa_step_h = gsa_measure(L, nat, hip, dev, sp, cfg, args.gsa_slots,
                                 max(5, args.steps // 5), "bf16")

    if args.copy_calibration:
        # 1 GiB each: a bf16 fill (writes only), three copies (the scale points) and three
        # max-reductions (reads only) of the same buffer, the latter two as checks of the
        # copy's scale factors
        nbytes = 1 << 30
        a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        for _ in range(3):
            a.amax()
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {nbytes} B copies, 3 x {nbytes} B reductions",
              file=sys.stderr, flush=True)

    e = 2 if cfg.dtype == "bf16" else 4
    mode_s = args.state_mode
    print(f"[bench] {cfg.name}: {ms_per_step:.4f} ms/step (HIP events, timed steps; "
          f"{wall * 1e3 / args.steps:.4f} ms wall incl. the cache flush), warm cache "
          f"{warm_ms:.4f} ms/step; profiling pass "
          f"with every stage boundary recorded: {traced_ms:.4f} ms/step wall, "
          f"{gpu_ms_from_events:.4f} ms (sum of stage events)", file=sys.stderr)
    print(f"{'pass':4s} {'stage':16s} {'us':>9s} {'GB/s':>8s} {'TFLOP/s':>8s}", file=sys.stderr)
    for (tag, name), ms in stages.items():
        if ms <= 0.0:   # a stage with no launch for this shape
            continue
        byt, fl = stage_work(name, tag, mode_s, B, H, T, dk, dv, C, e, train and tag == "fwd")
        print(f"{tag:4s} {name:16s} {ms * 1e3:9.2f} {byt / ms / 1e6:8.0f} {fl / ms / 1e9:8.1f}",
              file=sys.stderr)
    print(f"[bench] {dom_key[0]}:{dom_key[1]} in the timed steps: {dom_ms * 1e3:.2f} us",
          file=sys.stderr)
    byt, fl = stage_work(dom_key[1], dom_key[0], mode_s, B, H, T, dk, dv, C, e,
                         train and dom_key[0] == "fwd")
    ai = fl / byt if byt else float("inf")
    ridge = PEAK_BF16 / PEAK_HBM
    if ai < ridge:
        roof = {"bound": "hbm", "achieved": byt / (dom_ms * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": fl / (dom_ms * 1e-3) / 1e12, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    # the training pair's forward runs the intra-chunk kernel's fp32-operand instance
    ikey = lambda tag: "intra_save" if train and tag == "fwd" else f"intra_{tag}"  # noqa: E731
    kind = mode_s if (train or mode_s == "materialized" or fwd_only) else "recompute_pair"
    stage_key = ikey(dom_key[0]) if dom_key[1] == "intra" else dom_key[1]
    roof["traffic"] = counter_traffic(stage_key, cfg.name, kind)
    roof["kernel"] = f"{dom_key[0]}:{dom_key[1]}"
    roof["avg_launch_us"] = dom_ms * 1e3
    roof["algorithmic_bytes_per_launch"] = byt
    roof["algorithmic_flops_per_launch"] = fl
    roof["ai_flop_per_byte"] = ai
    # measured matrix-unit use (committed counter summary of the default gate options):
    # the dominant stage's busy fraction, and every MFMA stage's alongside
    mf = counter_mfma(cfg.name, kind) if not (args.scalar_gates or args.diag == "bf16") else {}
    roof["mfma_busy_frac"] = mf.get(stage_key, {}).get("mfma_busy_frac")
    roof["mfma_counters"] = mf or None
    # the intra-chunk kernel against the bf16 MFMA peak: its algorithmic flops over its live
    # duration (profiling pass), and the counters' busy fraction where they match
    intra_mfma = {}
    for tag in ("fwd", "bwd"):
        ms_i = stages.get((tag, "intra"), 0.0)
        if ms_i > 0.0:
            _, fl_i = stage_work("intra", tag, mode_s, B, H, T, dk, dv, C, e, train and tag == "fwd")
            intra_mfma[tag] = {"us": ms_i * 1e3, "tflops": fl_i / ms_i / 1e9,
                               "bf16_peak_frac": fl_i / (ms_i * 1e-3) / PEAK_BF16,
                               "mfma_busy_frac": mf.get(ikey(tag), {}).get("mfma_busy_frac")}

    tokens = B * T
    value = tokens / (ms_per_step * 1e-3)
    flops = path_flops(B, H, T, dk, dv, C, fwd_only)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": metric_name(cfg, fwd_only), "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name + ("_scalar_gates" if args.scalar_gates else "")
                   + ("_diag_bf16" if args.diag == "bf16" else ""),
                   "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": C,
                   "subchunk": cfg.subchunk, "state_mode": mode_s,
                   "pair": "train" if train else "recompute", "global_batch": B,
                   "seq_len": T, "parallelism": "none (1 GPU)"},
        "tflops": tflops, "mfma_peak_frac": flops / (ms_per_step * 1e-3) / PEAK_BF16,
        "roofline": roof,
        "intra_mfma": intra_mfma or None,
        "cache_flushed": flush,
        "cache_flush": "512 MiB write then 512 MiB read before each timed step, untimed" if flush else None,
        "warm_cache": warm_rec,
        "recompute_pair_step" if train else "train_pair_step": other_pair,
        "gate_logits_step": gate_fe,
        "scalar_gate_step": scalar_fe,
        "gsa_step": gsa_step,
        "gsa_step_bf16": gsa_step_h,
    }
    for arr in evf + evb + ev_dom + ev_step:
        hip.destroy(arr)
    if not args.no_decode:
        out["decode_step"] = decode_measure(L, nat, hip, dev, sp, H, dk, dv)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on host cores", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(d, cfg, min(args.cpu_tokens, T))
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
