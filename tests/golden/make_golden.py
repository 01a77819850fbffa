"""Writes tests/golden/tiny_oracle_case.json: a tiny seeded case and the oracle's outputs.

The pages print no worked example for this layer, so this fixture is a regression pin of
the oracle itself (its correctness is pinned separately by tests/test_oracle_pins.py).
Only the oracle is called.  Run:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import recurrence_fwd, recurrence_bwd  # noqa: E402


def main():
    rng = np.random.default_rng(20231211)
    B, H, T, dk, dv = 1, 2, 7, 3, 2
    q = np.round(rng.standard_normal((B, H, T, dk)), 3)
    k = np.round(rng.standard_normal((B, H, T, dk)), 3)
    v = np.round(rng.standard_normal((B, H, T, dv)), 3)
    la = -np.round(np.abs(rng.standard_normal((B, H, T, dk))) * 0.5, 3)
    S0 = np.round(rng.standard_normal((B, H, dk, dv)), 3)
    dO = np.round(rng.standard_normal((B, H, T, dv)), 3)
    dST = np.round(rng.standard_normal((B, H, dk, dv)), 3)
    o, ST = recurrence_fwd(q, k, v, la, S0)
    dq, dk_, dv_, dla, dS0 = recurrence_bwd(q, k, v, la, dO, S0, dST)
    arrays = dict(q=q, k=k, v=v, log_alpha=la, S0=S0, dO=dO, dS_T=dST, o=o, S_T=ST,
                  dq=dq, dk=dk_, dv=dv_, dlog_alpha=dla, dS0=dS0)
    doc = {
        "citation": "No worked example is printed on the pages; oracle regression pin. "
                    "Recurrence: 'Gated Linear Attention Transformers with Hardware-Efficient "
                    "Training' (atlas.scime.ai summary), Approach (gate G_t = alpha_t^T 1).",
        "generator": "tests/golden/make_golden.py (calls oracle.recurrence only)",
        "arrays": {k2: np.asarray(a).tolist() for k2, a in arrays.items()},
    }
    with open(os.path.join(HERE, "tiny_oracle_case.json"), "w") as fh:
        json.dump(doc, fh, indent=None, separators=(",", ":"))
        fh.write("\n")


if __name__ == "__main__":
    main()
