"""CPU fp64 oracle for chunkwise gated linear attention (GLA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its Python
binding) imports, calls or links this package; only the tests, the smoke check and the
CPU-baseline leg of the benchmark do.  It shares no code with the HIP path.

What it computes (page "Gated Linear Attention Transformers with Hardware-Efficient
Training", atlas.scime.ai summary, section Approach): a linear-attention recurrent state
S (dk x dv per batch and head) updated with a data-dependent low-rank gate
G_t = alpha_t^T 1, i.e. every row d of the state is decayed by alpha_t[d] in (0,1)
before the new key/value outer product is added; the output reads the updated state.

    S_t = diag(alpha_t) S_{t-1} + k_t^T v_t,     o_t = q_t S_t,     S_{-1} = S0.

Modules
  recurrence  plain step-by-step forward, its direct reverse-mode backward, the
              quadratic (parallel) form for tiny inputs, and the pages' closed-form
              gate gradient.
  chunkwise   fp64 chunkwise form (gate log-cumsum, inter-chunk states, intra-chunk
              products with two-level sub-chunking, chunk backward), exposing the
              intermediates for per-stage checks.
  gates       the gate front-end: log_alpha = logsigmoid(x) / tau from gate logits x, and
              the chain rule back to x.
  scalar      scalar-gate variants (one gate per token, or a constant decay per head):
              the layer with the gate repeated over the key dimension, its gradient
              summed back, and the parallel decay-matrix form used to pin it.
  gsa         Gated Slot Attention: the slot recurrence with a softmax read, its gradient
              by fp64 autograd of that recurrence, and the two-GLA-pass form.
  compare     error metrics used by the parity tests.

Every function is pinned by the CPU tests in tests/test_oracle_*.py against facts that do
not come from the oracle itself (closed forms, a library routine, finite differences,
torch autograd on an independent fp64 graph, exact rational arithmetic).
"""
from . import recurrence, chunkwise, compare, gates, scalar, gsa  # noqa: F401
from .recurrence import (recurrence_fwd, recurrence_bwd, quadratic_fwd,  # noqa: F401
                         closed_form_gate_grad)
