"""Seeded synthetic inputs for the chunkwise GLA layer, shared by the oracle tests,
the GPU parity tests and the benchmark.

This module holds the input recipe only (shapes, value distributions, seeds, rounding
of the inputs to their storage dtype). It performs none of the layer's arithmetic.

Workload shapes follow the layer sizes of the GLA Transformer paper summary
("Gated Linear Attention Transformers with Hardware-Efficient Training", atlas.scime.ai
summary, Key results / Measured effects: 340M and 1.3B models trained on 2K contexts,
extrapolation beyond 20K tokens). The gate logits g are turned into log-gates with
log_alpha = logsigmoid(g) / 16, a stand-in for the data-dependent low-rank gate of the
Approach section (the pages do not print the gate's parameterisation).

Draw order (one numpy PCG64 stream per config): g, q, k, v, dO, each drawn in float64
over its full [B,H,T,d] shape; q, k, v are scaled by 1/sqrt(dk); all values are cast
to float32 and then, for bf16 configs, rounded to bf16 (round-to-nearest-even).
The float64 views returned here hold exactly the values the device sees.

Scalar gates (one per token and head, the pages' scalar-gate ablation) come from a second
stream seeded (seed, 1), so that adding them changes none of the draws above: logits
g_s ~ N(gate_mean, 1) over [B,H,T], log_alpha_scalar = logsigmoid(g_s) / 16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["GlaConfig", "CONFIGS", "generate", "generate_gsa", "round_to_bf16_bits", "bf16_bits_to_f64",
           "logsigmoid"]


@dataclasses.dataclass(frozen=True)
class GlaConfig:
    name: str
    dtype: str            # "f32" or "bf16": storage/arithmetic dtype of q,k,v,log_alpha,o,...
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    subchunk: int = 16
    gate_mean: float = 0.0   # g ~ N(gate_mean, 1)
    seed: int = 0
    bwd: bool = True

    @property
    def tokens(self) -> int:
        return self.B * self.T

    def replace(self, **kw) -> "GlaConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  Unstated fields (sub-chunk 16, seed 0, chunk 64 for the long
# sequence) take the plainest choice.
CONFIGS = {
    "tiny_f32": GlaConfig("tiny_f32", "f32", 1, 1, 256, 64, 64, 64),
    "gla340m_t2k": GlaConfig("gla340m_t2k", "bf16", 8, 4, 2048, 128, 256, 64),
    "gla1p3b_t2k": GlaConfig("gla1p3b_t2k", "bf16", 4, 4, 2048, 256, 512, 64),
    "long_t20k": GlaConfig("long_t20k", "bf16", 1, 4, 20480, 256, 512, 64, gate_mean=2.0,
                           bwd=False),
}
for _T in (1024, 4096, 8192):
    for _C in (64, 128):
        CONFIGS[f"sweep_t{_T}_c{_C}"] = GlaConfig(
            f"sweep_t{_T}_c{_C}", "bf16", 16384 // _T, 4, _T, 256, 512, _C, gate_mean=-3.0)


def logsigmoid(x: np.ndarray) -> np.ndarray:
    """log(1/(1+exp(-x))) computed without overflow."""
    return -np.logaddexp(0.0, -x)


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns (uint16), round-to-nearest-even, via float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _quantize(x: np.ndarray, dtype: str):
    """Returns (storage array, exact float64 values)."""
    x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "bf16":
        bits = round_to_bf16_bits(x32)
        return bits, bf16_bits_to_f64(bits)
    raise ValueError(dtype)


def generate(cfg: GlaConfig, *, with_dO: bool = True, T: int | None = None):
    """Draws one config's inputs.

    Returns a dict with, for each of q, k, v, log_alpha (and dO): `X` (float64, the exact
    values) and `X_store` (float32 array or uint16 bf16 bits, what goes to the device).
    `T` overrides the sequence length (for reduced-size parity cases).
    """
    T = cfg.T if T is None else T
    rng = np.random.default_rng(cfg.seed)
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    out = {}
    g = rng.standard_normal((B, H, T, dk)) + cfg.gate_mean
    la = logsigmoid(g) / 16.0
    inv = 1.0 / math.sqrt(dk)
    q = rng.standard_normal((B, H, T, dk)) * inv
    k = rng.standard_normal((B, H, T, dk)) * inv
    v = rng.standard_normal((B, H, T, dv)) * inv
    # the raw gate logits too, for the gate front-end (log_alpha formed from them)
    items = [("log_alpha", la), ("gate_logits", g), ("q", q), ("k", k), ("v", v)]
    if with_dO:
        items.append(("dO", rng.standard_normal((B, H, T, dv))))
    rng_s = np.random.default_rng([cfg.seed, 1])
    gsc = rng_s.standard_normal((B, H, T)) + cfg.gate_mean
    items += [("log_alpha_scalar", logsigmoid(gsc) / 16.0), ("gate_logits_scalar", gsc)]
    for name, arr in items:
        store, exact = _quantize(arr, cfg.dtype)
        out[name + "_store"] = store
        out[name] = exact
    return out


def generate_gsa(cfg: GlaConfig, m: int, *, with_dO: bool = True):
    """Inputs of Gated Slot Attention with m slots: q, k, v (and dO) exactly as `generate`
    draws them, plus per-slot gates from a third stream seeded (seed, 2): logits
    g_slot ~ N(gate_mean, 1) over [B,H,T,m] and log_alpha_slot = logsigmoid(g_slot) / 8."""
    out = generate(cfg, with_dO=with_dO)
    rng = np.random.default_rng([cfg.seed, 2])
    g = rng.standard_normal((cfg.B, cfg.H, cfg.T, m)) + cfg.gate_mean
    store, exact = _quantize(logsigmoid(g) / 8.0, cfg.dtype)
    out["log_alpha_slot_store"] = store
    out["log_alpha_slot"] = exact
    return out
