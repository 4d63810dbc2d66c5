"""Comparison helpers shared by the tests (no method arithmetic here)."""
from __future__ import annotations

import numpy as np


def as_f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def rowwise_rel(x, y, floor=1e-30):
    """max over rows of ||x_row - y_row||_inf / ||y_row||_inf (last axis = row).

    This is the error metric of the parity tests: per (b,h,t) vector for
    o, k~, d; per (b,h) matrix for the state (flatten the last two axes first).
    """
    x = as_f64(x)
    y = as_f64(y)
    assert x.shape == y.shape, (x.shape, y.shape)
    if x.size == 0:
        return 0.0
    num = np.max(np.abs(x - y), axis=-1)
    den = np.maximum(np.max(np.abs(y), axis=-1), floor)
    return float(np.max(num / den))


def matrix_rel(x, y, floor=1e-30):
    """Per-matrix max-abs relative error over the last two axes, max over matrices."""
    x = as_f64(x)
    y = as_f64(y)
    return rowwise_rel(x.reshape(x.shape[:-2] + (-1,)), y.reshape(y.shape[:-2] + (-1,)), floor)


def max_abs(x, y):
    x = as_f64(x)
    y = as_f64(y)
    return float(np.max(np.abs(x - y))) if x.size else 0.0
