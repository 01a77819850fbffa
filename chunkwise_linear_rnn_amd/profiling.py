"""Summaries of rocprofv3 output for this library's kernels (text, a few KB).

    python -m chunkwise_linear_rnn_amd.profiling stats <run_kernel_stats.csv> "<command>"
    python -m chunkwise_linear_rnn_amd.profiling counters <FETCH csv> <WRITE csv> <copy bytes> \
        <stage> <workload> "<commands>"

`stats` renders the per-kernel table of a `rocprofv3 --kernel-trace --stats` run.
`counters` turns two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --copy-calibration` into HBM bytes per launch of one stage: the counters are
scaled so that the plain 1 GiB device copy in the same run reads and writes exactly its
size; the result is written as JSON (matched by bench.py against the kernel source hash).
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys

STAGE_KERNEL = {"bwd_chunk": "k_bwd_chunk", "bwd_dqk_dv": "k_bwd_dqk_dv",
                "fwd_fused": "k_fwd_fused", "intra": "k_intra",
                "state_scan_fwd": "k_state_scan", "state_scan_rev": "k_state_scan",
                "state_scans": "k_state_scan", "seg_state": "k_state_scan",
                "output": "k_output", "gate_cumsum": "k_gate_cumsum", "gate_grad": "k_gate_grad",
                "gate_tot": "k_gate_tot", "gate_reduce": "k_gate_reduce", "state_dot": "k_state_dot",
                "state_scan": "k_state_scan"}
STAGE_SOURCE = {"bwd_chunk": "k_bwd.hip", "bwd_dqk_dv": "k_bwd.hip",
                "fwd_fused": "k_fwd.hip", "intra": "k_intra.hip",
                "state_scan_fwd": "k_state.hip", "state_scan_rev": "k_state.hip",
                "state_scans": "k_state.hip", "seg_state": "k_state.hip",
                "output": "k_fwd.hip", "gate_cumsum": "k_gate.hip", "gate_grad": "k_gate.hip",
                "gate_tot": "k_gate.hip", "gate_reduce": "k_gate.hip", "state_dot": "k_gate.hip",
                "state_scan": "k_state.hip"}


# Stages whose kernel name is shared by several launches of a step: the template
# arguments that pick the stage's instance (mangled, or demangled, symbol text).
STAGE_SYMBOL = {"state_scans": ("ELi1ELb1E", ", 1, true"),     # stores states, cross terms
                "seg_state": ("ELi0ELb0E", ", 0, false")}      # midpoint state only


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
    return {"stage": stage, "workload": workload,
            "source_sha256": source_digest(stage, root),
            "fetch_kib_raw": sum(kf) / len(kf), "write_kib_raw": sum(kw) / len(kw),
            "copy_scale_fetch": sf, "copy_scale_write": sw,
            "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
            "traffic_bytes_per_launch": fetch + write, "launches": len(kf), "command": command}


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        sys.stdout.write(stats_table(sys.argv[2], sys.argv[3]))
    elif sys.argv[1] == "counters":
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        rec = counters(sys.argv[2], sys.argv[3], float(sys.argv[4]), sys.argv[5], sys.argv[6],
                       sys.argv[7], root)
        print(json.dumps(rec, indent=1))
