"""Row gather (embedding lookup) and its VJP, a scatter-add, in fp64 -- test
infrastructure.

Source: "Backprop for kernel writers", section 06 "Top-k & routing": a
selection y_m = x[i_m] passes gradient only to the selected slots, so the
backward is the scatter-add  xbar_j = sum over m with i_m = j of ybar_m  (zero
for rows never selected); with distinct indices (top-k) a plain scatter
suffices, with repeated indices (gather, embedding lookup) every duplicate
must be summed -- a plain scatter keeps only one of them -- and atomic adds
make the result order-dependent.  Section 04 "The duality": a value read by
many outputs sums their gradients.

Here x is a table [V, D], idx [M] integer rows, y [M, D] = x[idx].  An index
outside [0, V) is not defined by the pages; reading taken: it selects nothing
(its y row is zero), contributes nothing to the gradient and is counted.

:func:`sorted_order` is the stable order by index (equal indices keep
increasing m) in which the HIP path sums each row's contributions; it is a
plain argsort, stated here so tests can check the permutation exactly.
"""
from __future__ import annotations

import numpy as np


def valid_mask(idx, V):
    idx = np.asarray(idx, np.int64)
    return (idx >= 0) & (idx < V)


def fwd(x, idx):
    """y[m] = x[idx[m]] (zero row for an index outside [0, V))."""
    x = np.asarray(x, np.float64)
    idx = np.asarray(idx, np.int64)
    V = x.shape[0]
    ok = valid_mask(idx, V)
    y = np.zeros((idx.size, x.shape[1]), np.float64)
    y[ok] = x[idx[ok]]
    return y


def bwd(dy, idx, V, dx_old=None):
    """dx[v] = sum over m with idx[m] = v of dy[m], in increasing m; returns
    (dx [V, D], n_invalid).  With dx_old the sum is added into it."""
    dy = np.asarray(dy, np.float64)
    idx = np.asarray(idx, np.int64)
    dx = np.zeros((V, dy.shape[1]), np.float64) if dx_old is None else np.array(dx_old, np.float64)
    n_invalid = 0
    for m in range(idx.size):
        v = idx[m]
        if 0 <= v < V:
            dx[v] += dy[m]
        else:
            n_invalid += 1
    return dx, n_invalid


def sorted_order(idx, V):
    """Positions m sorted by idx[m] (stable), invalid indices last (in m order)."""
    idx = np.asarray(idx, np.int64)
    key = np.where(valid_mask(idx, V), idx, V)
    return np.argsort(key, kind="stable")


def counts(idx, V):
    """Number of m selecting each row v."""
    idx = np.asarray(idx, np.int64)
    ok = valid_mask(idx, V)
    return np.bincount(idx[ok], minlength=V)
