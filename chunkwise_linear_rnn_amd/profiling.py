"""Summaries of rocprofv3 output for this library's kernels (text, a few KB).

    python -m chunkwise_linear_rnn_amd.profiling stats <run_kernel_stats.csv> "<command>"
    python -m chunkwise_linear_rnn_amd.profiling counters <FETCH csv> <WRITE csv> <copy bytes> \
        <stage> <workload> "<commands>"

`stats` renders the per-kernel table of a `rocprofv3 --kernel-trace --stats` run.
`counters` turns two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --copy-calibration` into HBM bytes per launch of one stage: the counters are
scaled so that the plain 1 GiB device copy in the same run reads and writes exactly its
size, and the factors that a read-only and a write-only kernel of the same size would
give are reported beside them as checks; the result is written as JSON (matched by
bench.py against the kernel source hash).

    python -m chunkwise_linear_rnn_amd.profiling mfma <counter csv> <workload> "<command>"

`mfma` turns one `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16
GRBM_GUI_ACTIVE` run into per-kernel matrix-unit figures (JSON, keyed by stage where the
kernel belongs to one, with the kernel source hash): bf16 MFMA work per launch
(MOPS x 512 flop), the busy fraction of the 1024 SIMDs' matrix units over the launch
(busy cycles / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)) and the achieved fraction of the
2.5 PFLOP/s bf16 peak at 2.4 GHz.

    python -m chunkwise_linear_rnn_amd.profiling valu <counter csv> <workload> "<command>"

`valu` turns one `rocprofv3 --pmc` run of the counters in VALU_COUNTERS into per-kernel
instruction mixes (JSON, like `mfma`): vector-ALU, transcendental, matrix, LDS and scalar
instructions per wave, and the share of the SIMDs' cycles that the vector-ALU issue takes.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys

STAGE_KERNEL = {"bwd_dqk_dv": "k_bwd_dqk_dv",
                "fwd_fused": "k_fwd_fused", "intra": "k_intra",
                "state_scan_fwd": "k_state_scan", "state_scan_rev": "k_state_scan",
                "state_scans": "k_state_scan", "seg_state": "k_state_scan",
                "output": "k_output",
                "gate_tot": "k_gate_tot", "gate_reduce": "k_gate_reduce", "state_dot": "k_state_dot",
                "state_scan": "k_state_scan", "intra_fwd": "k_intra", "intra_bwd": "k_intra",
                "intra_save": "k_intra"}
STAGE_SOURCE = {"bwd_dqk_dv": "k_bwd.hip",
                "fwd_fused": "k_fwd.hip", "intra": "k_intra.hip",
                "state_scan_fwd": "k_state.hip", "state_scan_rev": "k_state.hip",
                "state_scans": "k_state.hip", "seg_state": "k_state.hip",
                "output": "k_fwd.hip",
                "gate_tot": "k_gate.hip", "gate_reduce": "k_gate.hip", "state_dot": "k_gate.hip",
                "state_scan": "k_state.hip", "intra_fwd": "k_intra.hip", "intra_bwd": "k_intra.hip",
                "intra_save": "k_intra.hip"}


# Stages whose kernel name is shared by several launches of a step: the template
# arguments that pick the stage's instance (mangled, or demangled, symbol text).
STAGE_SYMBOL = {"state_scans": ("ELi1ELb1E", ", 1, true"),     # stores states, cross terms
                "seg_state": ("ELi0ELb0E", ", 0, false"),      # segment end states only
                "state_scan": ("ELi2ELb0E", ", 2, false"),     # materialized forward states
                # the forward's intra-chunk kernel writes Kh^T in bf16, the backward's in fp32;
                # the training pair's forward (which keeps the backward's operands) runs the
                # backward's instance
                "intra_fwd": ("DF16bDF16bDF16bLi", "bf16, bf16, bf16,"),
                "intra_bwd": ("DF16bDF16bfLi", "bf16, bf16, float,"),
                "intra_save": ("DF16bDF16bfLi", "bf16, bf16, float,")}


def matches(stage: str, name: str) -> bool:
    if STAGE_KERNEL[stage] not in name:
        return False
    keys = STAGE_SYMBOL.get(stage)
    return keys is None or any(k in name for k in keys)


def code_text(src: str) -> bytes:
    """The source with comments removed and whitespace collapsed: what the compiler sees."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return " ".join(src.split()).encode()


def source_digest(stage: str, root: str) -> str:
    """sha256 over the code (comments aside) of the stage's kernel source and the shared
    device headers it includes."""
    h = hashlib.sha256()
    csrc = os.path.join(root, "chunkwise_linear_rnn_amd", "csrc")
    for f in (STAGE_SOURCE[stage], "gla_common.cuh", "gla_gate.cuh", "gla_internal.h"):
        h.update(code_text(open(os.path.join(csrc, f)).read()))
    return h.hexdigest()


def short(name: str) -> str:
    m = re.search(r"(k_[a-z_]+)", name)
    return m.group(1) if m else name[:40]


def stats_table(path: str, command: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = [f"command: {command}", "",
           f"{'kernel':18s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'share%':>7s}  symbol"]
    for r in rows:
        out.append(f"{short(r['Name']):18s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                   f"{float(r['Percentage']):7.2f}  {r['Name'][:90]}")
    return "\n".join(out) + "\n"


def _counter_rows(path, counter):
    rows = list(csv.DictReader(open(path)))
    key = next(k for k in rows[0] if k.lower() in ("counter_value", "value"))
    name_key = next(k for k in rows[0] if k.lower() in ("kernel_name", "kernel-name", "name"))
    cname = next(k for k in rows[0] if k.lower() in ("counter_name", "counter"))
    return [(r[name_key], float(r[key])) for r in rows if r[cname] == counter]


def counters(fetch_csv, write_csv, copy_bytes, stage, workload, command, root):
    f = _counter_rows(fetch_csv, "FETCH_SIZE")
    w = _counter_rows(write_csv, "WRITE_SIZE")
    # the calibration copy (a device-to-device buffer copy); the fill that initializes its
    # source writes but reads nothing, so it is not a calibration point
    def is_copy(n):
        n = n.lower()
        return "copy" in n and "fill" not in n
    copy_f = [v for n, v in f if is_copy(n)]
    copy_w = [v for n, v in w if is_copy(n)]
    kf = [v for n, v in f if matches(stage, n)]
    kw = [v for n, v in w if matches(stage, n)]
    if stage in ("state_scan_fwd", "state_scan_rev"):   # two launches per step: keep one of each pair
        kf, kw = kf[0::2] if stage.endswith("fwd") else kf[1::2], kw[0::2] if stage.endswith("fwd") else kw[1::2]
    sf = copy_bytes / (1024.0 * (sum(copy_f) / len(copy_f)))
    sw = copy_bytes / (1024.0 * (sum(copy_w) / len(copy_w)))
    fetch = sum(kf) / len(kf) * 1024.0 * sf
    write = sum(kw) / len(kw) * 1024.0 * sw
    # checks of the two factors on kernels of the same size that only read (the bf16
    # max-reductions) or only write (the bf16 fill of the copy's source); the cache flush
    # of the timed steps fills uint8 and sums float32, so it matches neither
    red_f = [v for n, v in f if "reduce" in n.lower() and "bfloat16" in n.lower()
             and ("maxnan" in n.lower() or "maxops" in n.lower())]
    fill_w = [v for n, v in w if "fill" in n.lower() and "bfloat16" in n.lower()]
    check_f = copy_bytes / (1024.0 * (sum(red_f) / len(red_f))) if red_f else None
    check_w = copy_bytes / (1024.0 * max(fill_w)) if fill_w else None
    return {"stage": stage, "workload": workload,
            "source_sha256": source_digest(stage, root),
            "fetch_kib_raw": sum(kf) / len(kf), "write_kib_raw": sum(kw) / len(kw),
            "copy_scale_fetch": sf, "copy_scale_write": sw,
            "read_only_scale_fetch": check_f, "write_only_scale_write": check_w,
            "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
            "traffic_bytes_per_launch": fetch + write, "launches": len(kf), "command": command}


MFMA_STAGES = ("fwd_fused", "bwd_dqk_dv", "state_scans", "seg_state", "output",
               "state_scan", "intra_fwd", "intra_bwd", "intra_save")
SIMDS, XCDS, CLOCK_HZ, PEAK_BF16 = 1024, 8, 2.4e9, 2.5e15


def mfma(path, workload, command, root):
    """Per-kernel MFMA figures (averages per launch) from one counter run."""
    rows = list(csv.DictReader(open(path)))
    agg = {}
    for r in rows:
        d = agg.setdefault(r["Kernel_Name"], {})
        d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    kernels = []
    for name, d in agg.items():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in d or "GRBM_GUI_ACTIVE" not in d:
            continue
        mean = {c: sum(v) / len(v) for c, v in d.items()}
        cycles = mean["GRBM_GUI_ACTIVE"] / XCDS
        busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"]
        flop = mean.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512.0
        secs = cycles / CLOCK_HZ
        kernels.append({"kernel": short(name), "symbol": name[:120],
                        "launches": len(d["GRBM_GUI_ACTIVE"]),
                        "gpu_cycles_per_launch": cycles, "mfma_busy_cycles": busy,
                        "mfma_busy_frac": busy / (cycles * SIMDS) if cycles else 0.0,
                        "bf16_gflop_per_launch": flop / 1e9,
                        "bf16_tflops": flop / secs / 1e12 if secs else 0.0,
                        "bf16_peak_frac": flop / secs / PEAK_BF16 if secs else 0.0,
                        "stages": [st for st in MFMA_STAGES if matches(st, name)]})
    kernels.sort(key=lambda k: -k["gpu_cycles_per_launch"] * k["launches"])
    digests = {st: source_digest(st, root) for st in MFMA_STAGES}
    return {"workload": workload, "command": command, "source_sha256": digests,
            "kernels": kernels}


VALU_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA", "SQ_INSTS_LDS",
                 "SQ_INSTS_SALU", "SQ_WAVES", "GRBM_GUI_ACTIVE")


def valu(path, workload, command, root):
    """Per-kernel instruction mix (averages per launch) from one counter run of
    VALU_COUNTERS: instructions per wave, and the share of the 1024 SIMDs' cycles over the
    launch that issuing the vector-ALU instructions takes, counting 4 cycles per wave64
    instruction and 16 per transcendental (matrix instructions are not vector-ALU issue
    here and are left out)."""
    rows = list(csv.DictReader(open(path)))
    agg = {}
    for r in rows:
        d = agg.setdefault(r["Kernel_Name"], {})
        d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    kernels = []
    for name, d in agg.items():
        if any(c not in d for c in VALU_COUNTERS):
            continue
        mean = {c: sum(v) / len(v) for c, v in d.items()}
        cycles = mean["GRBM_GUI_ACTIVE"] / XCDS
        waves = max(mean["SQ_WAVES"], 1.0)
        vec = mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"]
        trans = mean["SQ_INSTS_VALU_TRANS_F32"]
        issue = 4.0 * (vec - trans) + 16.0 * trans
        kernels.append({"kernel": short(name), "symbol": name[:120],
                        "launches": len(d["GRBM_GUI_ACTIVE"]),
                        "gpu_cycles_per_launch": cycles, "waves": mean["SQ_WAVES"],
                        "valu_per_wave": vec / waves, "trans_per_wave": trans / waves,
                        "mfma_per_wave": mean["SQ_INSTS_MFMA"] / waves,
                        "lds_per_wave": mean["SQ_INSTS_LDS"] / waves,
                        "salu_per_wave": mean["SQ_INSTS_SALU"] / waves,
                        "valu_issue_frac": issue / (cycles * SIMDS) if cycles else 0.0,
                        "stages": [st for st in MFMA_STAGES if matches(st, name)]})
    kernels.sort(key=lambda k: -k["gpu_cycles_per_launch"] * k["launches"])
    digests = {st: source_digest(st, root) for st in MFMA_STAGES}
    return {"workload": workload, "command": command, "source_sha256": digests,
            "kernels": kernels}


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        sys.stdout.write(stats_table(sys.argv[2], sys.argv[3]))
    elif sys.argv[1] == "counters":
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        rec = counters(sys.argv[2], sys.argv[3], float(sys.argv[4]), sys.argv[5], sys.argv[6],
                       sys.argv[7], root)
        print(json.dumps(rec, indent=1))
    elif sys.argv[1] == "mfma":
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        print(json.dumps(mfma(sys.argv[2], sys.argv[3], sys.argv[4], root), indent=1))
    elif sys.argv[1] == "valu":
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        print(json.dumps(valu(sys.argv[2], sys.argv[3], sys.argv[4], root), indent=1))
