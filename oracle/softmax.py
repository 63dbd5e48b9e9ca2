"""Row softmax and its VJP, in fp64 -- test infrastructure.

Source: "Backprop for kernel writers", section 01 "The only idea" (the
backward returns the vector-Jacobian product and never forms the Jacobian)
and the softmax section after 04 "The duality": the dense softmax Jacobian
diag(y) - y y^T applied to dy collapses to one row scalar s = sum_j dy_j y_j
and the elementwise dx_j = y_j (dy_j - s); the backward needs y, not x; the
max shift of the forward is free because softmax is shift invariant.

Save-the-statistics form (same section: y can be recomputed from the saved
max and logsumexp; section 07 "Fusion": keep only L = m + log l per row and
rebuild p = exp(x - L)): :func:`lse` is L and :func:`bwd_from_x` is the same
VJP with y rebuilt exactly from x.
"""
from __future__ import annotations

import numpy as np


def fwd(x: np.ndarray) -> np.ndarray:
    """y[r, j] = exp(x[r, j] - m_r) / sum_k exp(x[r, k] - m_r), m_r = max_k x[r, k]."""
    x = np.asarray(x, np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def bwd(dy: np.ndarray, y: np.ndarray) -> np.ndarray:
    """dx[r, j] = y[r, j] * (dy[r, j] - s_r), s_r = sum_k dy[r, k] * y[r, k].

    ``y`` is whatever the forward saved (for a bf16 forward, the bf16 values).
    """
    dy = np.asarray(dy, np.float64)
    y = np.asarray(y, np.float64)
    s = np.sum(dy * y, axis=-1, keepdims=True)
    return y * (dy - s)


def lse(x: np.ndarray) -> np.ndarray:
    """L_r = m_r + log sum_k exp(x[r, k] - m_r), m_r = max_k x[r, k]."""
    x = np.asarray(x, np.float64)
    m = np.max(x, axis=-1)
    return m + np.log(np.sum(np.exp(x - m[..., None]), axis=-1))


def bwd_from_x(dy: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The softmax VJP with y = softmax(x) rebuilt from the forward's input."""
    return bwd(dy, fwd(x))
