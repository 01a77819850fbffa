"""Tensor-level wrappers over the C ABI.  Argument marshalling only: shapes and dtypes
are checked, outputs and the workspace are allocated with torch on the inputs' device,
and raw pointers plus torch's current HIP stream go to libgla_mi355x.so."""
from __future__ import annotations

import ctypes

import torch

from ._native import (BF16, DIAG_BF16, DIAG_F32, F32, GATE_LOG_ALPHA, GATE_LOGITS,
                      GATE_PER_KEY, GATE_SCALAR,
                      MATERIALIZED, RECOMPUTE, PASS_BWD, PASS_FWD, PASS_STATES, PASS_FWD_SAVE,
                      PASS_BWD_SAVED, saved_bytes, GlaError, lib,
                      make_desc, make_gsa_desc, gsa_workspace_bytes, workspace_bytes)

_DT = {torch.float32: F32, torch.bfloat16: BF16}
_MODES = {"materialized": MATERIALIZED, "recompute": RECOMPUTE}
_DIAGS = {"f32": DIAG_F32, "bf16": DIAG_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _desc_from(q, v, chunk, subchunk, state_mode, gate_tau=None, scalar=False, diag="f32"):
    """gate_tau: None when the log_alpha argument is log_alpha itself, else the temperature
    of gate logits (log_alpha = logsigmoid(x) / gate_tau).  scalar: one gate per token
    ([B, H, T]) instead of one per key dimension.  diag: arithmetic of the diagonal
    intra-chunk sub-blocks, "f32" (default) or "bf16" (opt-in, bf16 inputs)."""
    if diag not in _DIAGS:
        raise ValueError(f"diag must be one of {sorted(_DIAGS)}")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, H, T, d]")
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    mode = _MODES[state_mode] if isinstance(state_mode, str) else int(state_mode)
    shape = GATE_SCALAR if scalar else GATE_PER_KEY
    if gate_tau is None:
        return make_desc(B, H, T, dk, dv, chunk, subchunk, _DT[q.dtype], mode,
                         gate_shape=shape, diag=_DIAGS[diag])
    return make_desc(B, H, T, dk, dv, chunk, subchunk, _DT[q.dtype], mode, GATE_LOGITS,
                     float(gate_tau), shape, _DIAGS[diag])


def _is_scalar(log_alpha):
    """A [B, H, T] gate (one per token) rather than [B, H, T, dk]."""
    return isinstance(log_alpha, torch.Tensor) and log_alpha.dim() == 3


def _gate_shape(log_alpha, B, H, T, dk):
    return (B, H, T) if _is_scalar(log_alpha) else (B, H, T, dk)


def _ws_buffer(need, device, workspace):
    """(buffer, its size in bytes): the caller's workspace after checking its device,
    layout and size, or a fresh one of `need` bytes.  The real size goes to the C ABI,
    which checks it against what the call needs."""
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != device:
            raise ValueError(f"workspace must be a tensor on {device}")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        size = workspace.numel() * workspace.element_size()
        if size < need:
            raise ValueError(f"workspace must hold at least {need} bytes on {device} "
                             f"(it holds {size})")
        return workspace, size
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device), need


def _workspace(desc, pass_, device, workspace):
    return _ws_buffer(workspace_bytes(desc, pass_), device, workspace)


def _call(name, st):
    if st != 0:
        raise GlaError(st, name)


def fwd(q, k, v, log_alpha, S0=None, *, chunk=64, subchunk=16, state_mode="recompute",
        final_state=True, workspace=None, gate_tau=None, diag="f32"):
    """o, S_T = the GLA layer forward (S_T is None when final_state is False).
    gate_tau: when set, log_alpha holds gate logits x and the layer uses
    logsigmoid(x) / gate_tau.  log_alpha [B, H, T] (instead of [B, H, T, dk]) is a scalar
    gate per token, shared by every key dimension.  diag: "f32" or "bf16" diagonal
    intra-chunk sub-blocks."""
    desc, o, S_T = _fwd_args(q, k, v, log_alpha, S0, chunk, subchunk, state_mode, gate_tau,
                             diag, final_state)
    dev = q.device
    ws, need = _workspace(desc, PASS_FWD, dev, workspace)
    _call("gla_chunk_fwd", lib().gla_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                               _ptr(log_alpha), _ptr(S0), _ptr(o), _ptr(S_T),
                                               _ptr(ws), need, _stream(dev)))
    return o, S_T


def _fwd_args(q, k, v, log_alpha, S0, chunk, subchunk, state_mode, gate_tau, diag,
              final_state):
    desc = _desc_from(q, v, chunk, subchunk, state_mode, gate_tau, _is_scalar(log_alpha), diag)
    dev, dt = q.device, q.dtype
    B, H, T, dk, dv = desc.B, desc.H, desc.T, desc.dk, desc.dv
    for t, n, shp in ((q, "q", (B, H, T, dk)), (k, "k", (B, H, T, dk)),
                      (v, "v", (B, H, T, dv)),
                      (log_alpha, "log_alpha", _gate_shape(log_alpha, B, H, T, dk))):
        _check(t, n, shp, dt, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if final_state else None
    return desc, o, S_T


def fwd_save(q, k, v, log_alpha, S0=None, *, chunk=64, subchunk=16, final_state=True,
             workspace=None, saved=None, gate_tau=None, diag="f32"):
    """o, S_T, saved: the recomputed-states forward of fwd (gla_chunk_fwd_save) that also
    keeps the backward's intra-chunk operands in `saved` (a uint8 device tensor of at least
    saved_bytes(desc) bytes, allocated when None) for bwd_saved with the same inputs."""
    desc, o, S_T = _fwd_args(q, k, v, log_alpha, S0, chunk, subchunk, RECOMPUTE, gate_tau,
                             diag, final_state)
    dev = q.device
    ws, need = _workspace(desc, PASS_FWD_SAVE, dev, workspace)
    sv, sneed = _ws_buffer(saved_bytes(desc), dev, saved)
    _call("gla_chunk_fwd_save", lib().gla_chunk_fwd_save(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(S0), _ptr(o),
        _ptr(S_T), _ptr(sv), sneed, _ptr(ws), need, _stream(dev)))
    return o, S_T, sv


def check_gates(q, v, log_alpha, *, gate_tau=None):
    """The number of elements of log_alpha that break the layer's precondition (finite and
    <= 0; gate logits with gate_tau: finite), counted on the device (gla_check_gates;
    synchronizes the stream).  Shapes and options as for fwd."""
    desc = _desc_from(q, v, 64, 16, RECOMPUTE, gate_tau, _is_scalar(log_alpha))
    dev = q.device
    B, H, T, dk = desc.B, desc.H, desc.T, desc.dk
    _check(log_alpha, "log_alpha", _gate_shape(log_alpha, B, H, T, dk), q.dtype, dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    n = ctypes.c_int64(0)
    _call("gla_check_gates", lib().gla_check_gates(ctypes.byref(desc), _ptr(log_alpha), _ptr(ws),
                                                   256, ctypes.byref(n), _stream(dev)))
    return int(n.value)


def bwd(q, k, v, log_alpha, dO, S0=None, dS_T=None, *, chunk=64, subchunk=16,
        want_dS0=True, workspace=None, gate_tau=None, diag="f32"):
    """dq, dk, dv, dlog_alpha, dS0 for the loss gradient (dO, dS_T).  With gate_tau set
    (gate logits in log_alpha) the fourth output is the gradient with respect to them.
    A scalar gate (log_alpha [B, H, T]) gets its gradient summed over the key dimension."""
    desc, outs = _bwd_args(q, k, v, log_alpha, dO, S0, dS_T, chunk, subchunk, gate_tau, diag,
                           want_dS0)
    dq, dk_, dv_, dla, dS0 = outs
    dev = q.device
    ws, need = _workspace(desc, PASS_BWD, dev, workspace)
    _call("gla_chunk_bwd", lib().gla_chunk_bwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(S0), _ptr(dO),
        _ptr(dS_T), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dS0), _ptr(ws), need,
        _stream(dev)))
    return dq, dk_, dv_, dla, dS0


def _bwd_args(q, k, v, log_alpha, dO, S0, dS_T, chunk, subchunk, gate_tau, diag, want_dS0):
    desc = _desc_from(q, v, chunk, subchunk, RECOMPUTE, gate_tau, _is_scalar(log_alpha), diag)
    dev, dt = q.device, q.dtype
    B, H, T, dk, dv = desc.B, desc.H, desc.T, desc.dk, desc.dv
    for t, n, shp in ((q, "q", (B, H, T, dk)), (k, "k", (B, H, T, dk)),
                      (v, "v", (B, H, T, dv)),
                      (log_alpha, "log_alpha", _gate_shape(log_alpha, B, H, T, dk)),
                      (dO, "dO", (B, H, T, dv))):
        _check(t, n, shp, dt, dev)
    for t, n in ((S0, "S0"), (dS_T, "dS_T")):
        if t is not None:
            _check(t, n, (B, H, dk, dv), torch.float32, dev)
    dq = torch.empty_like(q)
    dk_ = torch.empty_like(k)
    dv_ = torch.empty_like(v)
    dla = torch.empty_like(log_alpha)
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if want_dS0 else None
    return desc, (dq, dk_, dv_, dla, dS0)


def bwd_saved(q, k, v, log_alpha, dO, saved, S0=None, dS_T=None, *, chunk=64, subchunk=16,
              want_dS0=True, workspace=None, gate_tau=None, diag="f32"):
    """bwd from the intra-chunk operands that fwd_save kept in `saved` for the same q, k,
    log_alpha and options (gla_chunk_bwd_saved): the same results, without the backward's
    intra-chunk kernel."""
    desc, outs = _bwd_args(q, k, v, log_alpha, dO, S0, dS_T, chunk, subchunk, gate_tau, diag,
                           want_dS0)
    dq, dk_, dv_, dla, dS0 = outs
    dev = q.device
    need_s = saved_bytes(desc)
    if (not isinstance(saved, torch.Tensor) or saved.device != dev or not saved.is_contiguous()
            or saved.numel() * saved.element_size() < need_s):
        raise ValueError(f"saved must be the contiguous buffer of fwd_save on {dev} "
                         f"(at least {need_s} bytes)")
    ws, need = _workspace(desc, PASS_BWD_SAVED, dev, workspace)
    _call("gla_chunk_bwd_saved", lib().gla_chunk_bwd_saved(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(S0), _ptr(dO),
        _ptr(dS_T), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla), _ptr(dS0), _ptr(saved),
        saved.numel() * saved.element_size(), _ptr(ws), need, _stream(dev)))
    return dq, dk_, dv_, dla, dS0


def gate_cumsum(log_alpha, chunk=64, gate_tau=None, dk=None):
    """g (chunk-local inclusive cumsum, fp32) and gamma (chunk totals, fp32).  A scalar
    gate (log_alpha [B, H, T]) needs dk: g and gamma are broadcast over it."""
    if log_alpha.dim() not in (3, 4) or log_alpha.dtype not in _DT:
        raise ValueError("log_alpha must be [B,H,T,dk] or [B,H,T] float32/bfloat16")
    scalar = log_alpha.dim() == 3
    if scalar:
        if dk is None:
            raise ValueError("a scalar gate needs dk")
        B, H, T = log_alpha.shape
    else:
        B, H, T, dk = log_alpha.shape
    shape = GATE_SCALAR if scalar else GATE_PER_KEY
    if gate_tau is None:
        desc = make_desc(B, H, T, dk, 64, chunk, 16, _DT[log_alpha.dtype], RECOMPUTE,
                         gate_shape=shape)
    else:
        desc = make_desc(B, H, T, dk, 64, chunk, 16, _DT[log_alpha.dtype], RECOMPUTE,
                         GATE_LOGITS, float(gate_tau), shape)
    _check(log_alpha, "log_alpha", tuple(log_alpha.shape), log_alpha.dtype, log_alpha.device)
    N = (T + chunk - 1) // chunk
    g = torch.empty((B, H, T, dk), dtype=torch.float32, device=log_alpha.device)
    gamma = torch.empty((B, H, N, dk), dtype=torch.float32, device=log_alpha.device)
    _call("gla_gate_cumsum", lib().gla_gate_cumsum(ctypes.byref(desc), _ptr(log_alpha), _ptr(g),
                                                   _ptr(gamma), _stream(log_alpha.device)))
    return g, gamma


def chunk_states(k, v, log_alpha, S0=None, *, chunk=64, subchunk=16, workspace=None,
                 gate_tau=None):
    """states [B,H,N,dk,dv] (state before every chunk, fp32) and S_T."""
    desc = _desc_from(k, v, chunk, subchunk, MATERIALIZED, gate_tau, _is_scalar(log_alpha))
    dev, dt = k.device, k.dtype
    B, H, T, dk, dv = desc.B, desc.H, desc.T, desc.dk, desc.dv
    for t, n, shp in ((k, "k", (B, H, T, dk)), (v, "v", (B, H, T, dv)),
                      (log_alpha, "log_alpha", _gate_shape(log_alpha, B, H, T, dk))):
        _check(t, n, shp, dt, dev)
    if S0 is not None:
        _check(S0, "S0", (B, H, dk, dv), torch.float32, dev)
    N = (T + chunk - 1) // chunk
    states = torch.empty((B, H, N, dk, dv), dtype=torch.float32, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws, need = _workspace(desc, PASS_STATES, dev, workspace)
    _call("gla_chunk_states", lib().gla_chunk_states(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(S0), _ptr(states), _ptr(S_T),
        _ptr(ws), need, _stream(dev)))
    return states, S_T


class GLAFunction(torch.autograd.Function):
    """Autograd wrapper.  Recomputed states (the default): forward gla_chunk_fwd_save,
    which keeps the backward's intra-chunk operands, and backward gla_chunk_bwd_saved from
    them (the chunk states are recomputed by the backward's scans).  Materialized states:
    forward gla_chunk_fwd, backward gla_chunk_bwd from the saved inputs.  The gate options
    of fwd / bwd (gate logits with gate_tau, a scalar gate per token, the diagonal
    precision) pass through; the gradient for log_alpha is then the one for what
    log_alpha holds."""

    @staticmethod
    def forward(ctx, q, k, v, log_alpha, S0, chunk, subchunk, state_mode, gate_tau, diag):
        if state_mode == "recompute":
            o, S_T, sv = fwd_save(q, k, v, log_alpha, S0, chunk=chunk, subchunk=subchunk,
                                  gate_tau=gate_tau, diag=diag)
        else:
            o, S_T = fwd(q, k, v, log_alpha, S0, chunk=chunk, subchunk=subchunk,
                         state_mode=state_mode, gate_tau=gate_tau, diag=diag)
            sv = None
        ctx.save_for_backward(q, k, v, log_alpha, S0, sv)
        ctx.cfg = (chunk, subchunk, gate_tau, diag)
        return o, S_T

    @staticmethod
    def backward(ctx, dO, dS_T):
        q, k, v, log_alpha, S0, sv = ctx.saved_tensors
        chunk, subchunk, gate_tau, diag = ctx.cfg
        dO = dO.contiguous() if dO is not None else q.new_zeros(q.shape[:-1] + (v.shape[-1],))
        dS_T = dS_T.contiguous() if dS_T is not None else None
        opts = dict(chunk=chunk, subchunk=subchunk, want_dS0=S0 is not None, gate_tau=gate_tau,
                    diag=diag)
        if sv is not None:
            dq, dk, dv, dla, dS0 = bwd_saved(q, k, v, log_alpha, dO, sv, S0, dS_T, **opts)
        else:
            dq, dk, dv, dla, dS0 = bwd(q, k, v, log_alpha, dO, S0, dS_T, **opts)
        return dq, dk, dv, dla, dS0, None, None, None, None, None


class GSAFunction(torch.autograd.Function):
    """Autograd wrapper of Gated Slot Attention: forward gla_gsa_fwd, backward gla_gsa_bwd
    (which recomputes the forward from the saved inputs)."""

    @staticmethod
    def forward(ctx, q, k, v, log_alpha):
        o = gsa_fwd(q, k, v, log_alpha)
        ctx.save_for_backward(q, k, v, log_alpha)
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, log_alpha = ctx.saved_tensors
        return gsa_bwd(q, k, v, log_alpha, dO.contiguous())


def decode(q, k, v, log_alpha, S, *, gate_tau=None):
    """o = the recurrent evaluation of T tokens (T typically 1), S (float32
    [B, H, dk, dv]) updated in place: S <- diag(exp(log_alpha_t)) S + k_t^T v_t,
    o_t = q_t S, for t in order.  gate_tau: log_alpha holds gate logits (see fwd)."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, H, T, d]")
    if q.dtype not in _DT:
        raise ValueError(f"unsupported dtype {q.dtype}")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    for t, n, shp in ((q, "q", (B, H, T, dk)), (k, "k", (B, H, T, dk)),
                      (v, "v", (B, H, T, dv)),
                      (log_alpha, "log_alpha", _gate_shape(log_alpha, B, H, T, dk))):
        _check(t, n, shp, dt, dev)
    _check(S, "S", (B, H, dk, dv), torch.float32, dev)
    desc = _desc_from(q, v, 64, 16, RECOMPUTE, gate_tau, _is_scalar(log_alpha))
    o = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    _call("gla_decode", lib().gla_decode(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(log_alpha), _ptr(S), _ptr(o), _stream(dev)))
    return o


def gla(q, k, v, log_alpha, S0=None, chunk=64, subchunk=16, state_mode="recompute",
        gate_tau=None, diag="f32"):
    """Differentiable GLA layer: returns (o, S_T); options as for fwd."""
    return GLAFunction.apply(q, k, v, log_alpha, S0, chunk, subchunk, state_mode, gate_tau, diag)


def _gsa_desc(q, v, log_alpha):
    if q.dim() != 4 or v.dim() != 4 or log_alpha.dim() != 4:
        raise ValueError("q, v and log_alpha must be [B, H, T, d]")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("Gated Slot Attention takes float32 or bfloat16 tensors")
    B, H, T, dk = q.shape
    return make_gsa_desc(B, H, T, dk, v.shape[-1], log_alpha.shape[-1],
                         F32 if q.dtype == torch.float32 else BF16)


def gsa_fwd(q, k, v, log_alpha, *, workspace=None):
    """o of Gated Slot Attention: key/value slots [slots, d] forgotten by the per-slot
    gates exp(log_alpha) [B, H, T, slots], written with weight 1 - alpha, read by
    softmax(slots_k q) (float32, or bfloat16 with the first pass in fp32)."""
    desc = _gsa_desc(q, v, log_alpha)
    dev = q.device
    B, H, T, dk, dv, m = desc.B, desc.H, desc.T, desc.dk, desc.dv, desc.slots
    for t, n, shp in ((q, "q", (B, H, T, dk)), (k, "k", (B, H, T, dk)), (v, "v", (B, H, T, dv)),
                      (log_alpha, "log_alpha", (B, H, T, m))):
        _check(t, n, shp, q.dtype, dev)
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    ws, need = _ws_buffer(gsa_workspace_bytes(desc, PASS_FWD), dev, workspace)
    _call("gla_gsa_fwd", lib().gla_gsa_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(log_alpha), _ptr(o), _ptr(ws), need, _stream(dev)))
    return o


def gsa_bwd(q, k, v, log_alpha, dO, *, workspace=None):
    """dq, dk, dv, dlog_alpha of Gated Slot Attention for the loss gradient dO."""
    desc = _gsa_desc(q, v, log_alpha)
    dev = q.device
    B, H, T, dk, dv, m = desc.B, desc.H, desc.T, desc.dk, desc.dv, desc.slots
    for t, n, shp in ((q, "q", (B, H, T, dk)), (k, "k", (B, H, T, dk)), (v, "v", (B, H, T, dv)),
                      (log_alpha, "log_alpha", (B, H, T, m)), (dO, "dO", (B, H, T, dv))):
        _check(t, n, shp, q.dtype, dev)
    dq, dk_, dv_, dla = (torch.empty_like(x) for x in (q, k, v, log_alpha))
    ws, need = _ws_buffer(gsa_workspace_bytes(desc, PASS_BWD), dev, workspace)
    _call("gla_gsa_bwd", lib().gla_gsa_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(log_alpha), _ptr(dO), _ptr(dq), _ptr(dk_),
                                           _ptr(dv_), _ptr(dla), _ptr(ws), need, _stream(dev)))
    return dq, dk_, dv_, dla


def gsa(q, k, v, log_alpha):
    """Differentiable Gated Slot Attention: returns o (see gsa_fwd)."""
    return GSAFunction.apply(q, k, v, log_alpha)
