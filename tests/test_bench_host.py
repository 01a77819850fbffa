"""Host-side checks of bench.py's bookkeeping (no GPU): its algorithmic work model covers
every stage the library reports for the measured configurations, the dominant kernel's
per-launch figures at the 1.3B shape stay the documented ones, and the committed HBM
counter summaries belong to the current kernel sources."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def native():
    import chunkwise_linear_rnn_amd._native as nat
    if not os.path.exists(nat.lib_path()):
        from chunkwise_linear_rnn_amd.build import build
        build(verbose=False)
    nat.lib()   # host-only calls below: stage names, no launches
    return nat


@pytest.mark.parametrize("mode", ["recompute", "materialized"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk", [64, 128])
def test_every_traced_stage_has_a_work_model(bench, native, mode, dtype, chunk):
    sm = native.RECOMPUTE if mode == "recompute" else native.MATERIALIZED
    dt = native.BF16 if dtype == "bf16" else native.F32
    e = 2 if dtype == "bf16" else 4
    d = native.make_desc(4, 4, 2048, 256, 512, chunk, 16, dt, sm)
    for pass_, tag in ((native.PASS_FWD, "fwd"), (native.PASS_BWD, "bwd")):
        for with_dst in (False, True) if tag == "bwd" else (False,):
            for name in native.trace_stages(d, pass_, with_dst):
                byt, fl = bench.stage_work(name, tag, mode, 4, 4, 2048, 256, 512, chunk, e)
                if name == "seg_state" and dtype == "f32":
                    assert (byt, fl) == (0, 0)   # no sequence split in fp32: nothing launched
                    continue
                assert byt > 0, (tag, name)
                assert fl >= 0, (tag, name)
    if mode != "recompute":
        return
    # the training pair (recompute state mode only): its forward keeps the backward's
    # operands, whose backward has no intra-chunk stage
    for pass_, tag in ((native.PASS_FWD_SAVE, "fwd"), (native.PASS_BWD_SAVED, "bwd")):
        names = native.trace_stages(d, pass_)
        if tag == "bwd":
            assert "intra" not in names
        for name in names:
            byt, fl = bench.stage_work(name, tag, mode, 4, 4, 2048, 256, 512, chunk, e,
                                       tag == "fwd")
            if name == "seg_state" and dtype == "f32":
                continue
            assert byt > 0, (tag, name)
            if tag == "fwd" and dtype == "bf16":
                # the kept operands: Qh^T and Kh^T in fp32 (4 bytes a key element) on top
                # of what the plain forward writes; the later kernels read the split
                # Kh^T's high part alone
                plain, _ = bench.stage_work(name, tag, mode, 4, 4, 2048, 256, 512, chunk, e)
                tokp = 16 * ((2048 + chunk - 1) // chunk) * chunk
                extra = {"intra": 2 * tokp * 256 * 4}
                assert byt - plain == extra.get(name, 0), name


def test_dominant_kernel_figures_at_1p3b(bench):
    # one launch of the backward chunk kernel at B=4, H=4, T=2048, dk=256, dv=512, C=64, bf16
    byt, fl = bench.stage_work("bwd_dqk_dv", "bwd", "recompute", 4, 4, 2048, 256, 512, 64, 2)
    assert (byt, fl) == (491257856, 28991029248)


@pytest.mark.parametrize("stage", ["bwd_dqk_dv", "state_scans", "fwd_fused", "seg_state",
                                   "gate_tot"])
def test_counter_summaries_match_sources(bench, stage):
    """A summary taken on other kernel sources is not used: bench.py reports its traffic
    as null (checked here by the digest), until the counters are taken again."""
    path = os.path.join(ROOT, "profiles", f"counters_{stage}_gla1p3b_t2k.json")
    if not os.path.exists(path):
        pytest.skip(f"no counter summary for {stage}")
    if bench.counter_traffic(stage, "gla1p3b_t2k") is None:
        pytest.skip(f"{os.path.basename(path)} predates the current kernel sources "
                    "(bench.py reports its traffic as null)")


def test_mfma_summary_is_well_formed(bench):
    """The committed matrix-unit summary at the 1.3B shape: fractions within [0, 1], the
    MFMA stages present, and bench.py reading them back while the sources match."""
    import json
    path = os.path.join(ROOT, "profiles", "mfma_gla1p3b_t2k.json")
    if not os.path.exists(path):
        pytest.skip("no matrix-unit summary")
    with open(path) as fh:
        rec = json.load(fh)
    stages = set()
    for k in rec["kernels"]:
        assert 0.0 <= k["mfma_busy_frac"] <= 1.0, k["kernel"]
        assert 0.0 <= k["bf16_peak_frac"] <= 1.0, k["kernel"]
        assert k["gpu_cycles_per_launch"] > 0, k["kernel"]
        stages.update(k["stages"])
    # the training pair's kernels (the forward runs the fp32-operand intra-chunk instance)
    assert {"bwd_dqk_dv", "fwd_fused", "state_scans", "seg_state", "intra_save"} <= stages
    got = bench.counter_mfma("gla1p3b_t2k", "recompute")
    if not got:
        pytest.skip("mfma_gla1p3b_t2k.json predates the current kernel sources")
    for st, v in got.items():
        assert st in stages and 0.0 <= v["mfma_busy_frac"] <= 1.0


def test_metric_names_the_workload_it_ran(bench):
    from gla_inputs import CONFIGS as WORKLOADS
    head = WORKLOADS["gla1p3b_t2k"]
    assert bench.metric_name(head, False) == bench.METRIC
    for name in ("sweep_t8192_c64", "gla340m_t2k", "long_t20k"):
        w = WORKLOADS[name]
        m = bench.metric_name(w, name == "long_t20k")
        assert name in m and f"T={w.T}" in m and "1.3B" not in m
    assert bench.metric_name(WORKLOADS["long_t20k"], True).startswith("GLA fwd tokens/s")
    # the headline shape run forward-only is not the headline metric either
    assert bench.metric_name(head, True) != bench.METRIC


def test_more_than_one_gpu_is_refused():
    """bench.py --gpus N with N > 1 exits with a message (one GPU only), before any GPU use."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout.strip() == ""
