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
