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


def partials(x: np.ndarray, dy: np.ndarray, block_rows: int, tiles: int | None = None) -> np.ndarray:
    """Stage-1 partial rows P[t, j] = sum over rows i of tile t of x[i, j] * dy[i].

    The rows are cut into blocks of ``block_rows`` consecutive rows (the last
    one may be shorter) and block b belongs to tile b mod ``tiles``.  With
    ``tiles`` left out it is the number of blocks, so tile t is the page's
    row tile [t * block_rows, min((t + 1) * block_rows, N)).  However the
    rows are dealt to tiles, summing P over t gives grad_w.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    n = x.shape[0]
    nblocks = n_tiles(n, block_rows)
    T = nblocks if tiles is None else int(tiles)
    P = np.zeros((T, x.shape[1]), np.float64)
    for b in range(nblocks):
        lo, hi = b * block_rows, min((b + 1) * block_rows, n)
        P[b % T] += np.sum(x[lo:hi] * dy[lo:hi, None], axis=0)
    return P
