"""Host-only checks of the C ABI (no GPU needed): the library loads, exports every
function include/gla.h declares, and its argument validation / workspace planning
behave as documented."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def native():
    import chunkwise_linear_rnn_amd._native as nat
    if not os.path.exists(nat.lib_path()):
        from chunkwise_linear_rnn_amd.build import build
        build(verbose=False)
    nat.lib()
    return nat


def _header_functions():
    src = open(os.path.join(ROOT, "include", "gla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gla_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(native):
    names = _header_functions()
    assert "gla_chunk_fwd" in names and "gla_chunk_bwd" in names
    h = native.lib()
    for n in names:
        assert hasattr(h, n), n
    assert set(names) == set(native.SIGNATURES)


def test_status_strings_and_version(native):
    assert native.status_string(0) == "GLA_OK"
    assert native.status_string(3) == "GLA_ERR_WORKSPACE"
    assert native.status_string(99) == "GLA_ERR_UNKNOWN"
    assert native.version() >= 100


def test_validation_codes(native):
    D = native.make_desc
    ok = D(2, 4, 2048, 256, 512, 64, 16, native.BF16, native.RECOMPUTE)
    assert native.validate(ok, native.PASS_FWD) == 0
    assert native.validate(ok, native.PASS_BWD) == 0
    assert native.lib().gla_validate(None, 0) == 1
    assert native.validate(ok, 7) == 1
    cases_invalid = [D(-1, 1, 8, 64, 64), D(1, 1, 8, 64, 64, 0), D(1, 1, 8, 64, 64, 64, 0),
                     D(1, 1, 8, 64, 64, 64, 24), D(1, 1, 8, 64, 64, 64, 16, 5),
                     D(1, 1, 8, 64, 64, 64, 16, 1, 9)]
    for d in cases_invalid:
        assert native.validate(d) == 1, d
    cases_unsup = [D(1, 1, 8, 64, 64, 32, 16), D(1, 1, 8, 64, 64, 64, 32), D(1, 1, 8, 96, 64),
                   D(1, 1, 8, 320, 64), D(1, 1, 8, 64, 96), D(1, 1, 8, 64, 2048),
                   D(1, 1, 8, 64, 64, 128, 16, native.F32), D(70000, 1, 8, 64, 64)]
    for d in cases_unsup:
        assert native.validate(d) == 2, d
    # empty problems are valid
    assert native.validate(D(0, 4, 100, 64, 64)) == 0
    assert native.validate(D(1, 1, 0, 64, 64)) == 0


def test_workspace_planning(native):
    D = native.make_desc
    d = D(4, 4, 2048, 256, 512, 64, 16, native.BF16, native.RECOMPUTE)
    rec = native.workspace_bytes(d, native.PASS_FWD)
    d.state_mode = native.MATERIALIZED
    mat = native.workspace_bytes(d, native.PASS_FWD)
    bwd = native.workspace_bytes(d, native.PASS_BWD)
    # materialized keeps every chunk state: B*H*N*dk*dv bf16 = 128 MiB at this shape, where
    # the recompute forward keeps one segment start state (B*H*dk*dv fp32 = 8 MiB)
    assert mat - rec >= 4 * 4 * 32 * 256 * 512 * 2 - 4 * 4 * 256 * 512 * 4
    assert bwd > mat
    assert native.workspace_bytes(d, native.PASS_STATES) > 0
    assert native.workspace_bytes(D(0, 4, 100, 64, 64), native.PASS_BWD) == 0
    with pytest.raises(native.GlaError):
        native.workspace_bytes(D(1, 1, 8, 64, 96), native.PASS_FWD)
    out = ctypes.c_size_t(0)
    assert native.lib().gla_workspace_bytes(ctypes.byref(d), 0, None) == 1
    assert native.lib().gla_workspace_bytes(ctypes.byref(d), 0, ctypes.byref(out)) == 0


def test_errors_before_any_launch(native):
    """Invalid calls return their code on the host without touching a device."""
    L = native.lib()
    D = native.make_desc
    bad = D(1, 1, 8, 64, 96)
    p = ctypes.c_void_p(16)
    assert L.gla_chunk_fwd(ctypes.byref(bad), p, p, p, p, None, p, None, p, 1 << 20, None) == 2
    good = D(1, 1, 64, 64, 64)
    # required pointer missing
    assert L.gla_chunk_fwd(ctypes.byref(good), None, p, p, p, None, p, None, p, 1 << 20, None) == 1
    # misaligned pointer
    q = ctypes.c_void_p(18)
    assert L.gla_chunk_fwd(ctypes.byref(good), q, p, p, p, None, p, None, p, 1 << 20, None) == 1
    # workspace too small / missing
    assert L.gla_chunk_fwd(ctypes.byref(good), p, p, p, p, None, p, None, p, 16, None) == 3
    assert L.gla_chunk_fwd(ctypes.byref(good), p, p, p, p, None, p, None, None, 0, None) == 3
    assert L.gla_chunk_bwd(ctypes.byref(good), p, p, p, p, None, None, None, p, p, p, p, None,
                           p, 1 << 30, None) == 1
    assert L.gla_gate_cumsum(ctypes.byref(good), None, p, p, None) == 1


def test_check_gates_errors_before_any_launch(native):
    """gla_check_gates refuses bad arguments on the host (its count itself needs a GPU)."""
    L = native.lib()
    good = native.make_desc(1, 1, 64, 64, 64)
    p = ctypes.c_void_p(16)
    n = ctypes.c_int64(-1)
    assert L.gla_check_gates(ctypes.byref(good), p, p, 256, None, None) == 1        # no n_bad
    assert L.gla_check_gates(ctypes.byref(good), None, p, 256, ctypes.byref(n), None) == 1
    assert L.gla_check_gates(ctypes.byref(good), ctypes.c_void_p(18), p, 256,
                             ctypes.byref(n), None) == 1                             # misaligned
    assert L.gla_check_gates(ctypes.byref(good), p, None, 0, ctypes.byref(n), None) == 3
    assert L.gla_check_gates(ctypes.byref(good), p, p, 4, ctypes.byref(n), None) == 3
    assert L.gla_check_gates(ctypes.byref(native.make_desc(1, 1, 8, 64, 96)), p, p, 256,
                             ctypes.byref(n), None) == 2                             # unsupported
    empty = native.make_desc(1, 1, 0, 64, 64)
    n.value = -1
    assert L.gla_check_gates(ctypes.byref(empty), None, None, 0, ctypes.byref(n), None) == 0
    assert n.value == 0


def test_decode_validation_before_any_launch(native):
    """gla_decode checks its own shape rules on the host (chunk fields are not used)."""
    L = native.lib()
    D = native.make_desc
    p = ctypes.c_void_p(16)
    # supported: dk, dv multiples of 32
    for dk, dv, code in ((48, 64, 2), (64, 48, 2), (288, 64, 2), (64, 1056, 2), (0, 64, 2)):
        d = D(1, 1, 1, dk, dv)
        assert L.gla_decode(ctypes.byref(d), p, p, p, p, p, p, None) == code, (dk, dv)
    d = D(1, 1, 1, 96, 96)
    assert L.gla_decode(None, p, p, p, p, p, p, None) == 1
    assert L.gla_decode(ctypes.byref(d), p, p, p, p, None, p, None) == 1     # S required
    assert L.gla_decode(ctypes.byref(d), p, p, p, p, p, None, None) == 1     # o required
    assert L.gla_decode(ctypes.byref(d), ctypes.c_void_p(20), p, p, p, p, p, None) == 1
    bad_dtype = D(1, 1, 1, 96, 96, 64, 16, 7)
    assert L.gla_decode(ctypes.byref(bad_dtype), p, p, p, p, p, p, None) == 1
    neg = D(1, -1, 1, 96, 96)
    assert L.gla_decode(ctypes.byref(neg), p, p, p, p, p, p, None) == 1
    # nothing to do: no pointer is looked at
    assert L.gla_decode(ctypes.byref(D(1, 1, 0, 96, 96)), None, None, None, None, None, None,
                        None) == 0
    assert L.gla_decode(ctypes.byref(D(0, 3, 5, 96, 96)), None, None, None, None, None, None,
                        None) == 0


def test_gate_front_end_fields(native):
    """gate: 0 (log_alpha given) or 1 (logits, temperature gate_tau > 0 and finite)."""
    D = native.make_desc
    ok = D(1, 1, 64, 64, 64, 64, 16, native.BF16, native.RECOMPUTE, native.GATE_LOGITS, 16.0)
    assert native.validate(ok) == 0 and native.validate(ok, native.PASS_BWD) == 0
    for gate, tau in ((2, 1.0), (-1, 1.0), (1, 0.0), (1, -3.0), (1, float("nan")),
                      (1, float("inf"))):
        d = D(1, 1, 64, 64, 64, 64, 16, native.BF16, native.RECOMPUTE, gate, tau)
        assert native.validate(d) == 1, (gate, tau)
        p = ctypes.c_void_p(16)
        assert native.lib().gla_decode(ctypes.byref(d), p, p, p, p, p, p, None) == 1
    # the temperature is ignored when the gates are given as log_alpha
    assert native.validate(D(1, 1, 64, 64, 64, 64, 16, native.BF16, native.RECOMPUTE, 0, 0.0)) == 0


def test_gate_shape_field(native):
    """gate_shape: 0 (one gate per key dimension) or 1 (one gate per token); anything else
    is an invalid argument.  Scalar gates add the sum over d as a last backward stage and,
    on the bf16 chunk-64 path, a small workspace for its per-block partial sums."""
    D = native.make_desc
    base = dict(chunk=64, subchunk=16, dtype=native.BF16, state_mode=native.RECOMPUTE)
    for shape in (native.GATE_PER_KEY, native.GATE_SCALAR):
        for gate, tau in ((native.GATE_LOG_ALPHA, 1.0), (native.GATE_LOGITS, 8.0)):
            d = D(2, 2, 300, 128, 64, gate=gate, gate_tau=tau, gate_shape=shape, **base)
            assert native.validate(d) == 0 and native.validate(d, native.PASS_BWD) == 0
    for bad in (2, -1, 7):
        d = D(1, 1, 64, 64, 64, gate_shape=bad, **base)
        assert native.validate(d) == 1, bad
        p = ctypes.c_void_p(16)
        assert native.lib().gla_decode(ctypes.byref(d), p, p, p, p, p, p, None) == 1
    per_key = D(4, 4, 2048, 256, 512, **base)
    sc = D(4, 4, 2048, 256, 512, gate_shape=native.GATE_SCALAR, **base)
    assert native.workspace_bytes(sc, native.PASS_BWD) == (
        native.workspace_bytes(per_key, native.PASS_BWD) + 4 * 4 * 2048 * (256 // 64) * 4)
    assert native.workspace_bytes(sc, native.PASS_FWD) == native.workspace_bytes(per_key, native.PASS_FWD)
    assert native.trace_stages(sc, native.PASS_BWD)[-1] == "gate_reduce"
    assert "gate_reduce" not in native.trace_stages(per_key, native.PASS_BWD)
    f32 = D(1, 2, 100, 64, 64, 64, 16, native.F32, native.RECOMPUTE, gate_shape=native.GATE_SCALAR)
    assert native.trace_stages(f32, native.PASS_BWD)[-2:] == ["bwd_dqk_dv", "gate_reduce"]


def test_gsa_descriptor_validation(native):
    """Gated Slot Attention: float32 only in this build; dk and slots in {64..256} by 64."""
    G = native.make_gsa_desc
    L = native.lib()
    assert L.gla_gsa_validate(ctypes.byref(G(2, 2, 300, 128, 192, 64))) == 0
    assert L.gla_gsa_validate(ctypes.byref(G(2, 2, 300, 128, 192, 64, native.BF16))) == 0
    assert L.gla_gsa_validate(ctypes.byref(G(2, 2, 300, 128, 192, 64, 7))) == 1
    for bad in ((1, 1, 64, 96, 64, 64), (1, 1, 64, 64, 64, 32), (1, 1, 64, 64, 96, 64),
                (1, 1, 64, 64, 64, 320)):
        assert L.gla_gsa_validate(ctypes.byref(G(*bad))) == 2, bad
    assert L.gla_gsa_validate(ctypes.byref(G(-1, 1, 64, 64, 64, 64))) == 1
    assert L.gla_gsa_validate(None) == 1
    assert native.gsa_workspace_bytes(G(0, 2, 64, 64, 64, 64)) == 0
    assert native.gsa_workspace_bytes(G(1, 2, 64, 64, 64, 64), native.PASS_BWD) > \
        native.gsa_workspace_bytes(G(1, 2, 64, 64, 64, 64), native.PASS_FWD) > 0
    # bf16: fp32 copies for the first pass, bf16 copies and gradients for the second
    hb = G(1, 2, 64, 64, 64, 64, native.BF16)
    assert native.gsa_workspace_bytes(hb, native.PASS_BWD) > \
        native.gsa_workspace_bytes(hb, native.PASS_FWD) > 0
    p = ctypes.c_void_p(16)
    # a missing workspace is reported before any launch
    assert L.gla_gsa_fwd(ctypes.byref(G(1, 1, 64, 64, 64, 64)), p, p, p, p, p, None, 0, None) == 3


def test_caller_workspace_is_checked(native):
    """A caller-provided workspace that is too small, on another device, or not contiguous
    is refused before any call (the real byte size goes to the C ABI otherwise)."""
    import torch
    from chunkwise_linear_rnn_amd.ops import _ws_buffer
    cpu = torch.device("cpu")
    with pytest.raises(ValueError):
        _ws_buffer(100, cpu, torch.empty(99, dtype=torch.uint8))
    with pytest.raises(ValueError):
        _ws_buffer(100, torch.device("cuda", 0), torch.empty(200, dtype=torch.uint8))
    with pytest.raises(ValueError):
        _ws_buffer(100, cpu, torch.empty(400, dtype=torch.uint8)[::2])
    buf, size = _ws_buffer(100, cpu, torch.empty(64, dtype=torch.float32))
    assert size == 256
    buf, size = _ws_buffer(100, cpu, None)
    assert size == 100 and buf.numel() == 100


def test_diag_field_validation(native):
    D = native.make_desc
    d = D(1, 1, 64, 64, 64, 64, 16, native.BF16, native.RECOMPUTE, diag=native.DIAG_BF16)
    assert native.validate(d) == 0
    d.diag = 2
    assert native.validate(d) == 1
    d.diag = -1
    assert native.validate(d) == 1


def test_noalloc_refuses_oversized_problem_on_host(native):
    """gla_chunk_fwd_noalloc refuses a forward whose workspace would exceed its fixed
    scratch array (GLA_ERR_WORKSPACE) before touching the device, and an invalid
    descriptor as gla_chunk_fwd does; the pointers below are never dereferenced."""
    D = native.make_desc
    big = D(16, 4, 8192, 256, 512, 64, 16, native.BF16, native.MATERIALIZED)
    assert native.workspace_bytes(big, native.PASS_FWD) > (128 << 20)
    p = ctypes.c_void_p(1 << 20)
    L = native.lib()
    assert L.gla_chunk_fwd_noalloc(ctypes.byref(big), p, p, p, p, None, p, None, None) == 3
    bad = D(1, 1, 64, 96, 64)
    assert L.gla_chunk_fwd_noalloc(ctypes.byref(bad), p, p, p, p, None, p, None, None) == 2
    assert L.gla_chunk_fwd_noalloc(None, p, p, p, p, None, p, None, None) == 1


def test_training_pair_planning_and_errors(native):
    """The saving forward and the backward from saved operands: the intra-chunk operands
    move from the workspaces to the saved buffer (sizes as laid out: A, Qh, Qh^T and Kh^T as
    fp32 words, Kh, e^gamma, each region 256-byte aligned); materialized states have no
    saving forward; a missing or short saved buffer is refused before any launch."""
    L = native.lib()
    D = native.make_desc
    al = lambda n: (n + 255) // 256 * 256
    B, H, T, dk, dv, C = 4, 4, 2048, 256, 512, 64
    d = D(B, H, T, dk, dv, C, 16, native.BF16, native.RECOMPUTE)
    rows = B * H * (T // C) * C
    A, op, op32, eg = (al(B * H * (T // C) * C * C * 2), al(rows * dk * 2), al(rows * dk * 4),
                       al(B * H * (T // C) * dk * 4))
    assert native.saved_bytes(d) == A + op + op32 + op + op32 + eg
    fwd, fwd_s = (native.workspace_bytes(d, native.PASS_FWD),
                  native.workspace_bytes(d, native.PASS_FWD_SAVE))
    bwd, bwd_s = (native.workspace_bytes(d, native.PASS_BWD),
                  native.workspace_bytes(d, native.PASS_BWD_SAVED))
    assert fwd - fwd_s == A + op + op + eg
    assert bwd - bwd_s == A + op32 + op + op32 + eg
    out = ctypes.c_size_t(0)
    assert L.gla_saved_bytes(ctypes.byref(d), None) == 1
    m = D(B, H, T, dk, dv, C, 16, native.BF16, native.MATERIALIZED)
    assert L.gla_saved_bytes(ctypes.byref(m), ctypes.byref(out)) == 2
    assert native.validate(m, native.PASS_FWD_SAVE) == 2
    assert native.validate(m, native.PASS_BWD_SAVED) == 0
    # stage lists: the saving forward has the recompute forward's, the backward from saved
    # operands the backward's without the intra-chunk kernel
    def names(pass_, dst):
        n = L.gla_trace_stages(ctypes.byref(d), pass_, dst, None, 0)
        arr = (ctypes.c_char_p * n)()
        L.gla_trace_stages(ctypes.byref(d), pass_, dst, arr, n)
        return [s.decode() for s in arr]
    assert names(native.PASS_FWD_SAVE, 0) == names(native.PASS_FWD, 0)
    assert names(native.PASS_BWD_SAVED, 0) == names(native.PASS_BWD, 0)[1:]
    assert names(native.PASS_BWD_SAVED, 1) == names(native.PASS_BWD, 1)[1:]
    assert L.gla_trace_stages(ctypes.byref(d), 5, 0, None, 0) == -1
    # refusals on the host: no saved buffer, a short one, a materialized descriptor
    small = D(1, 1, 64, 64, 64)
    p = ctypes.c_void_p(16)
    need = native.saved_bytes(small)
    ws = 1 << 30
    assert L.gla_chunk_fwd_save(ctypes.byref(small), p, p, p, p, None, p, None, None, 0, p, ws,
                                None) == 3
    assert L.gla_chunk_fwd_save(ctypes.byref(small), p, p, p, p, None, p, None, p, need - 1, p,
                                ws, None) == 3
    ms = D(1, 1, 64, 64, 64, 64, 16, native.BF16, native.MATERIALIZED)
    assert L.gla_chunk_fwd_save(ctypes.byref(ms), p, p, p, p, None, p, None, p, need, p, ws,
                                None) == 2
    assert L.gla_chunk_bwd_saved(ctypes.byref(small), p, p, p, p, None, p, None, p, p, p, p, None,
                                 None, 0, p, ws, None) == 3
    assert L.gla_chunk_bwd_saved(ctypes.byref(small), p, p, p, p, None, p, None, p, p, p, p, None,
                                 p, need - 1, p, ws, None) == 3
    q = ctypes.c_void_p(18)   # a misaligned saved buffer
    assert L.gla_chunk_bwd_saved(ctypes.byref(small), p, p, p, p, None, p, None, p, p, p, p, None,
                                 q, need, p, ws, None) == 1
