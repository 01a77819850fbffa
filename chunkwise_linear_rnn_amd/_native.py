"""ctypes view of the C ABI in include/gla.h (libgla_mi355x.so, built in-tree).

Nothing here touches a GPU: loading the library and the host-only entry points
(gla_validate, gla_workspace_bytes, gla_status_string, gla_version) work on a machine
without one.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libgla_mi355x.so"

F32, BF16 = 0, 1
GATE_LOG_ALPHA, GATE_LOGITS = 0, 1
GATE_PER_KEY, GATE_SCALAR = 0, 1
MATERIALIZED, RECOMPUTE = 0, 1
DIAG_F32, DIAG_BF16 = 0, 1
PASS_FWD, PASS_BWD, PASS_STATES, PASS_FWD_SAVE, PASS_BWD_SAVED = 0, 1, 2, 3, 4

# Every function include/gla.h declares, with its ctypes signature.
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


class GlaDesc(ctypes.Structure):
    _fields_ = [("B", _i32), ("H", _i32), ("T", _i32), ("dk", _i32), ("dv", _i32),
                ("chunk", _i32), ("subchunk", _i32), ("dtype", _i32), ("state_mode", _i32),
                ("gate", _i32), ("gate_tau", ctypes.c_float), ("gate_shape", _i32),
                ("diag", _i32)]

    def __repr__(self):
        return "GlaDesc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


class GsaDesc(ctypes.Structure):
    _fields_ = [("B", _i32), ("H", _i32), ("T", _i32), ("dk", _i32), ("dv", _i32),
                ("slots", _i32), ("dtype", _i32)]

    def __repr__(self):
        return "GsaDesc(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_PDESC = ctypes.POINTER(GlaDesc)
_PGSA = ctypes.POINTER(GsaDesc)
SIGNATURES = {
    "gla_status_string": (ctypes.c_char_p, [_i32]),
    "gla_version": (_i32, []),
    "gla_validate": (_i32, [_PDESC, _i32]),
    "gla_workspace_bytes": (_i32, [_PDESC, _i32, ctypes.POINTER(_sz)]),
    "gla_check_gates": (_i32, [_PDESC, _vp, _vp, _sz, ctypes.POINTER(ctypes.c_int64), _vp]),
    "gla_gate_cumsum": (_i32, [_PDESC, _vp, _vp, _vp, _vp]),
    "gla_chunk_states": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gla_chunk_fwd": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gla_chunk_bwd": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _sz, _vp]),
    "gla_chunk_fwd_noalloc": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "gla_saved_bytes": (_i32, [_PDESC, ctypes.POINTER(_sz)]),
    "gla_chunk_fwd_save": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _sz,
                                  _vp]),
    "gla_chunk_bwd_saved": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _vp, _sz, _vp, _sz, _vp]),
    "gla_decode": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "gla_gsa_validate": (_i32, [_PGSA]),
    "gla_gsa_workspace_bytes": (_i32, [_PGSA, _i32, ctypes.POINTER(_sz)]),
    "gla_gsa_fwd": (_i32, [_PGSA, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gla_gsa_bwd": (_i32, [_PGSA, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "gla_trace_stages": (_i32, [_PDESC, _i32, _i32, ctypes.POINTER(ctypes.c_char_p), _i32]),
    "gla_chunk_fwd_traced": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp,
                                    ctypes.POINTER(_vp), _i32]),
    "gla_chunk_bwd_traced": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _sz, _vp, ctypes.POINTER(_vp), _i32]),
    "gla_chunk_fwd_save_traced": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                         _vp, _sz, _vp, ctypes.POINTER(_vp), _i32]),
    "gla_chunk_bwd_saved_traced": (_i32, [_PDESC, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp,
                                          ctypes.POINTER(_vp), _i32]),
}

_lib = None


def lib_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it first "
                               "(python -m chunkwise_linear_rnn_amd.build)")
        h = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


class GlaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_string(code)}")


def status_string(code: int) -> str:
    return lib().gla_status_string(int(code)).decode()


def version() -> int:
    return int(lib().gla_version())


def make_desc(B, H, T, dk, dv, chunk=64, subchunk=16, dtype=BF16, state_mode=RECOMPUTE,
              gate=GATE_LOG_ALPHA, gate_tau=1.0, gate_shape=GATE_PER_KEY,
              diag=DIAG_F32) -> GlaDesc:
    return GlaDesc(B, H, T, dk, dv, chunk, subchunk, dtype, state_mode, gate, gate_tau,
                   gate_shape, diag)


def validate(desc: GlaDesc, pass_: int = PASS_FWD) -> int:
    return int(lib().gla_validate(ctypes.byref(desc), int(pass_)))


def trace_stages(desc: GlaDesc, pass_: int, with_dS_T: bool = False) -> list:
    n = int(lib().gla_trace_stages(ctypes.byref(desc), int(pass_), int(bool(with_dS_T)), None, 0))
    if n < 0:
        raise ValueError("bad descriptor or pass")
    names = (ctypes.c_char_p * n)()
    lib().gla_trace_stages(ctypes.byref(desc), int(pass_), int(bool(with_dS_T)), names, n)
    return [x.decode() for x in names]


def saved_bytes(desc: GlaDesc) -> int:
    """Bytes of the buffer gla_chunk_fwd_save fills for gla_chunk_bwd_saved."""
    out = _sz(0)
    st = lib().gla_saved_bytes(ctypes.byref(desc), ctypes.byref(out))
    if st != 0:
        raise GlaError(st, "gla_saved_bytes")
    return out.value


def workspace_bytes(desc: GlaDesc, pass_: int = PASS_FWD) -> int:
    out = _sz(0)
    st = lib().gla_workspace_bytes(ctypes.byref(desc), int(pass_), ctypes.byref(out))
    if st != 0:
        raise GlaError(st, "gla_workspace_bytes")
    return int(out.value)


def make_gsa_desc(B, H, T, dk, dv, slots, dtype=F32) -> GsaDesc:
    return GsaDesc(B, H, T, dk, dv, slots, dtype)


def gsa_workspace_bytes(desc: GsaDesc, pass_: int = PASS_FWD) -> int:
    n = _sz()
    st = int(lib().gla_gsa_workspace_bytes(ctypes.byref(desc), int(pass_), ctypes.byref(n)))
    if st != 0:
        raise GlaError(st, "gla_gsa_workspace_bytes")
    return int(n.value)
