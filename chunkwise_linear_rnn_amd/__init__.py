"""MI355X (gfx950) chunkwise gated linear attention: Python binding of libgla_mi355x.so.

The binding only marshals arguments: it checks tensor shapes/dtypes/devices, allocates
outputs and the workspace with torch, and passes raw device pointers plus the current
HIP stream to the C ABI declared in include/gla.h.  Every step of the computation runs
in the library's HIP kernels; there is no CPU or PyTorch fallback.  If the library is
not built, every call raises.

Entry points mirror the C ABI:
    fwd(q, k, v, log_alpha, S0=None, ...)              -> (o, S_T)
    bwd(q, k, v, log_alpha, dO, S0=None, dS_T=None)     -> (dq, dk, dv, dlog_alpha, dS0)
    gate_cumsum(log_alpha, chunk)                       -> (g, gamma)
    chunk_states(k, v, log_alpha, S0=None)              -> (states, S_T)
    workspace_bytes(desc, pass_), validate(desc, pass_), status_string(code)
and GLAFunction, a torch.autograd.Function over fwd/bwd.
"""
from __future__ import annotations

from ._native import (GlaDesc, GlaError, F32, BF16, MATERIALIZED, RECOMPUTE, PASS_FWD,  # noqa: F401
                      PASS_BWD, PASS_STATES, PASS_FWD_SAVE, PASS_BWD_SAVED, GATE_LOG_ALPHA, GATE_LOGITS, GATE_PER_KEY, GATE_SCALAR,
                      DIAG_F32, DIAG_BF16,
                      lib, lib_path, make_desc, make_gsa_desc, gsa_workspace_bytes, status_string,
                      trace_stages, saved_bytes,
                      validate, version, workspace_bytes)
from .ops import (fwd, bwd, fwd_save, bwd_saved, check_gates, gate_cumsum, chunk_states, decode, GLAFunction, gla,  # noqa: F401
                  GSAFunction, gsa, gsa_fwd, gsa_bwd)

__all__ = ["fwd", "bwd", "fwd_save", "bwd_saved", "saved_bytes", "check_gates", "gate_cumsum", "chunk_states", "decode", "GLAFunction", "gla", "GlaDesc",
           "GSAFunction", "gsa", "gsa_fwd", "gsa_bwd", "make_gsa_desc", "gsa_workspace_bytes",
           "GlaError", "make_desc", "workspace_bytes", "validate", "status_string", "version",
           "lib", "lib_path"]
