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
                assert byt > 0, (tag, name)
                assert fl >= 0, (tag, name)


def test_dominant_kernel_figures_at_1p3b(bench):
    # one launch of the backward chunk kernel at B=4, H=4, T=2048, dk=256, dv=512, C=64, bf16
    byt, fl = bench.stage_work("bwd_dqk_dv", "bwd", "recompute", 4, 4, 2048, 256, 512, 64, 2)
    assert (byt, fl) == (491257856, 28991029248)


@pytest.mark.parametrize("stage", ["bwd_dqk_dv", "state_scans", "fwd_fused", "seg_state",
                                   "gate_tot"])
def test_counter_summaries_match_sources(bench, stage):
    assert bench.counter_traffic(stage, "gla1p3b_t2k") is not None, (
        f"profiles/counters_{stage}_gla1p3b_t2k.json was taken on other kernel sources")
