"""Fused scaled-SiLU y = w * x * sigmoid(x) and its VJP, in fp64 -- test infrastructure.

Source: "Backward in Triton -- autograd.Function and the backward grid",
section "A complete minimal example -- fused scaled-SiLU, end to end":
w is one learnable scalar; with s = sigmoid(x) and silu = x * s, the
elementwise input gradient is dx = dy * w * (s + silu * (1 - s)) and the
scalar parameter gradient is dw = sum over all elements of dy * silu.
Section "fp32 accumulation, and why gradients use +=": an existing dw is
added into.
"""
from __future__ import annotations

import numpy as np


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)), evaluated without overflow on either side."""
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def fwd(x: np.ndarray, w: float) -> np.ndarray:
    """y = w * x * sigmoid(x)."""
    x = np.asarray(x, np.float64)
    return float(w) * x * sigmoid(x)


def bwd(dy: np.ndarray, x: np.ndarray, w: float, dw_old=None):
    """(dx, dw): dx = dy * w * (s + x s (1 - s)), dw = sum(dy * x * s) (+ dw_old)."""
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    s = sigmoid(x)
    dx = dy * float(w) * (s + x * s * (1.0 - s))
    dw = np.sum(dy * x * s)
    if dw_old is not None:
        dw = float(dw_old) + dw
    return dx, dw


def partials(dy: np.ndarray, x: np.ndarray, elems_per_tile: int) -> np.ndarray:
    """Stage-1 partials P[t] = sum over elements k of tile t of dy[k] * x[k] * s[k].

    Tile t holds elements [t * elems_per_tile, min((t + 1) * elems_per_tile, n)).
    """
    dy = np.asarray(dy, np.float64).reshape(-1)
    x = np.asarray(x, np.float64).reshape(-1)
    n = x.size
    T = -(-n // int(elems_per_tile))
    c = dy * x * sigmoid(x)
    return np.array([np.sum(c[t * elems_per_tile:min((t + 1) * elems_per_tile, n)])
                     for t in range(T)], np.float64)
