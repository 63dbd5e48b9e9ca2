"""Row-wise weighted sum y = x . w and its VJP, in fp64 -- test infrastructure.

Source: "Writing Triton Kernels with Autograd: A Minimal End-to-End Example",
section 1 "Problem Setup" (y[i] = sum_j x[i, j] * w[j], x [N, D], w [D],
y [N]), section 3 "Backward: Deriving Gradients First" (grad_x is the outer
product of grad_out with w; grad_w sums x * grad_out over the rows; the
two-stage strategy writes one partial row per tile of BLOCK_N rows and sums
those partial rows afterwards).  "Backward in Triton -- autograd.Function and
the backward grid", section "fp32 accumulation, and why gradients use +="
(an existing parameter gradient is added into, not overwritten).
"""
from __future__ import annotations

import numpy as np


def fwd(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[i] = sum_j x[i, j] * w[j]."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    return np.sum(x * w[None, :], axis=1)


def bwd(dy: np.ndarray, x: np.ndarray, w: np.ndarray, grad_w_old=None):
    """(grad_x, grad_w) for upstream gradient dy [N].

    grad_x[i, j] = dy[i] * w[j]; grad_w[j] = sum_i x[i, j] * dy[i];
    with ``grad_w_old`` given, grad_w is added into it.
    """
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    grad_x = dy[:, None] * w[None, :]
    grad_w = np.sum(x * dy[:, None], axis=0)
    if grad_w_old is not None:
        grad_w = np.asarray(grad_w_old, np.float64) + grad_w
    return grad_x, grad_w


def n_tiles(n_rows: int, rows_per_tile: int) -> int:
    """Number of row tiles: ceil(n_rows / rows_per_tile)."""
    return -(-int(n_rows) // int(rows_per_tile))


def partials(x: np.ndarray, dy: np.ndarray, rows_per_tile: int) -> np.ndarray:
    """Stage-1 partial rows P[t, j] = sum over rows i of tile t of x[i, j] * dy[i].

    Tile t holds rows [t * rows_per_tile, min((t + 1) * rows_per_tile, N)).
    Summing P over t gives grad_w.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    n = x.shape[0]
    T = n_tiles(n, rows_per_tile)
    P = np.zeros((T, x.shape[1]), np.float64)
    for t in range(T):
        lo, hi = t * rows_per_tile, min((t + 1) * rows_per_tile, n)
        P[t] = np.sum(x[lo:hi] * dy[lo:hi, None], axis=0)
    return P
