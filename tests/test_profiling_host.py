"""Host-side pieces of the profiling summaries (no GPU)."""
from chunkwise_linear_rnn_amd import profiling


def test_code_text_ignores_comments_and_spacing():
    a = "int x = 1;  // one\n/* block\n comment */ float y =\n  2.f;\n"
    b = "int x = 1;\nfloat y = 2.f; // two"
    assert profiling.code_text(a) == profiling.code_text(b) == b"int x = 1; float y = 2.f;"
    assert profiling.code_text("int x = 1;") != profiling.code_text("int x = 2;")


def test_stage_maps_cover_each_other():
    assert set(profiling.STAGE_KERNEL) == set(profiling.STAGE_SOURCE)
    for stage in profiling.STAGE_SYMBOL:
        assert stage in profiling.STAGE_KERNEL


def _csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, v in rows:
            f.write(f'"{name}",{counter},{v}\n')


def test_counter_scaling_and_its_checks(tmp_path):
    """The copy sets the scale; a read-only reduction and a write-only fill of the same
    size are reported as checks; the timed steps' cache flush (uint8 fill, float sum) and
    the stage's own kernels do not count as calibration points."""
    gib = 1 << 30
    kib = gib / 1024.0
    fetch = [("__amd_rocclr_copyBuffer", kib / 2), ("__amd_rocclr_copyBuffer", kib / 2),
             ("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<c10::BFloat16, "
              "at::native::func_wrapper_t<c10::BFloat16, at::native::MaxNanFunctor<"
              "c10::BFloat16> >, unsigned int, c10::BFloat16, 4, 4> >", kib / 2.5),
             ("void at::native::reduce_kernel<512, 1, at::native::ReduceOp<float, "
              "at::native::func_wrapper_t<float, at::native::sum_functor<float> > > >", 7.0),
             ("k_bwd_dqk_dv<__hip_bfloat16>", 1000.0), ("k_bwd_dqk_dv<__hip_bfloat16>", 3000.0)]
    write = [("__amd_rocclr_copyBuffer", kib), ("__amd_rocclr_copyBuffer", kib),
             ("void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<"
              "c10::BFloat16>, std::array<char*, 1ul> >", kib / 1.25),
             ("void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<"
              "unsigned char>, std::array<char*, 1ul> >", kib * 9),
             ("k_bwd_dqk_dv<__hip_bfloat16>", 500.0), ("k_bwd_dqk_dv<__hip_bfloat16>", 500.0)]
    fp, wp = tmp_path / "f.csv", tmp_path / "w.csv"
    _csv(fp, "FETCH_SIZE", fetch)
    _csv(wp, "WRITE_SIZE", write)
    r = profiling.counters(str(fp), str(wp), gib, "bwd_dqk_dv", "w", "cmd", ".")
    assert abs(r["copy_scale_fetch"] - 2.0) < 1e-12 and abs(r["copy_scale_write"] - 1.0) < 1e-12
    assert abs(r["read_only_scale_fetch"] - 2.5) < 1e-12
    assert abs(r["write_only_scale_write"] - 1.25) < 1e-12
    assert r["launches"] == 2
    assert abs(r["fetch_bytes_per_launch"] - 2000.0 * 1024 * 2.0) < 1e-6
    assert abs(r["write_bytes_per_launch"] - 500.0 * 1024) < 1e-6


def test_valu_instruction_mix(tmp_path):
    """Instructions per wave and the vector-ALU issue share: matrix instructions are taken
    out of the vector-ALU count, transcendentals take 16 cycles, the others 4, over the
    launch's cycles on 1024 SIMDs (GRBM_GUI_ACTIVE summed over 8 XCDs)."""
    name = "_ZN3gla7k_intraIDF16bDF16bDF16bLi64ELb1ELb0EEEv"
    vals = {"SQ_INSTS_VALU": [1100.0, 1300.0], "SQ_INSTS_VALU_TRANS_F32": [100.0, 100.0],
            "SQ_INSTS_MFMA": [200.0, 200.0], "SQ_INSTS_LDS": [50.0, 70.0],
            "SQ_INSTS_SALU": [10.0, 10.0], "SQ_WAVES": [4.0, 4.0],
            "GRBM_GUI_ACTIVE": [8.0 * 100.0, 8.0 * 100.0]}
    p = tmp_path / "v.csv"
    with open(p, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for c, vs in vals.items():
            for v in vs:
                f.write(f'"{name}",{c},{v}\n')
        f.write('"other_kernel",SQ_INSTS_VALU,5\n')   # a kernel without the full set: skipped
    r = profiling.valu(str(p), "w", "cmd", ".")
    assert len(r["kernels"]) == 1
    k = r["kernels"][0]
    assert k["launches"] == 2 and k["gpu_cycles_per_launch"] == 100.0
    assert k["valu_per_wave"] == (1200.0 - 200.0) / 4 and k["trans_per_wave"] == 25.0
    assert k["mfma_per_wave"] == 50.0 and k["lds_per_wave"] == 15.0
    issue = 4.0 * (1000.0 - 100.0) + 16.0 * 100.0
    assert abs(k["valu_issue_frac"] - issue / (100.0 * 1024)) < 1e-15
    assert k["stages"] == ["intra_fwd"]   # the forward variant (bf16 transposed operands)
