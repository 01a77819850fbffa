"""Error metrics for parity checks.  TEST INFRASTRUCTURE ONLY.

max_rel:  max_i |x_i - y_i| / max_i |y_i|   (infinity-norm relative error; an
          elementwise ratio is undefined where y_i = 0)
normwise: ||x - y||_2 / ||y||_2
Both fall back to the absolute error when the reference is identically zero.
"""
from __future__ import annotations

import numpy as np

__all__ = ["max_rel", "normwise", "report"]


def max_rel(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    if x.size == 0:
        return 0.0
    num = float(np.max(np.abs(x - y)))
    den = float(np.max(np.abs(y)))
    return num / den if den > 0 else num


def normwise(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    if x.size == 0:
        return 0.0
    num = float(np.linalg.norm((x - y).ravel()))
    den = float(np.linalg.norm(y.ravel()))
    return num / den if den > 0 else num


def report(x, y) -> dict:
    return {"max_rel": max_rel(x, y), "normwise": normwise(x, y)}
