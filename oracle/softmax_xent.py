"""Fused softmax-cross-entropy (mean over rows) forward and backward, in fp64.

Test infrastructure.  Source: "Backprop for kernel writers", section 02
"See it move" (softmax followed by cross-entropy: the two derivatives cancel
so the logit gradient is the softmax minus the one-hot of the true class)
and section 07 "Fusion" (store only L_r = m_r + log l_r, with m_r the row
max and l_r the row sum of exp(z - m_r); any probability is rebuilt as
exp(z - L_r)).

Definitions (R rows, C classes, target t_r):
  m_r      = max_j z[r, j]
  lse_r    = m_r + log sum_j exp(z[r, j] - m_r)
  loss_r   = lse_r - z[r, t_r]
  loss     = (1 / R) * sum_r loss_r
  dz[r, j] = grad_scale * (exp(z[r, j] - lse_r) - [j == t_r])

grad_scale is d(loss_total)/d(loss) / R; for the mean loss with unit upstream
gradient it is 1 / R.

Split form (section 07: the forward keeps only the row statistics and the
backward rebuilds p = exp(z - lse)): :func:`fwd` gives the loss and the
statistics; :func:`bwd` gives dz = (dloss / R) * (softmax(z) - onehot) for an
upstream gradient dloss of the mean loss.

Targets outside [0, C) are not defined by the pages.  Reading taken here:
such a row's loss is NaN (so is the mean), its logit gradient has no one-hot
term, and the rows are counted in ``n_invalid``.
"""
from __future__ import annotations

import numpy as np


def fwd_bwd(z: np.ndarray, targets: np.ndarray, grad_scale: float):
    """Returns dict(loss, row_loss, row_max, row_lse, dz, n_invalid)."""
    z = np.asarray(z, np.float64)
    t = np.asarray(targets, np.int64)
    R, C = z.shape
    m = np.max(z, axis=1)
    lse = m + np.log(np.sum(np.exp(z - m[:, None]), axis=1))
    valid = (t >= 0) & (t < C)
    rows = np.arange(R)
    z_t = np.where(valid, z[rows, np.where(valid, t, 0)], np.nan)
    row_loss = lse - z_t
    loss = np.sum(row_loss) / R if R > 0 else np.nan
    p = np.exp(z - lse[:, None])
    onehot = np.zeros_like(p)
    onehot[rows[valid], t[valid]] = 1.0
    dz = float(grad_scale) * (p - onehot)
    return {
        "loss": loss,
        "row_loss": row_loss,
        "row_max": m,
        "row_lse": lse,
        "dz": dz,
        "n_invalid": int(np.count_nonzero(~valid)),
    }


def fwd(z: np.ndarray, targets: np.ndarray):
    """Returns dict(loss, row_loss, row_max, row_lse, n_invalid) -- no gradient."""
    out = fwd_bwd(z, targets, 0.0)
    del out["dz"]
    return out


def bwd(z: np.ndarray, targets: np.ndarray, dloss: float) -> np.ndarray:
    """dz[r, j] = (dloss / R) * (softmax(z)[r, j] - [j == t_r]); no one-hot term
    for a target outside [0, C)."""
    z = np.asarray(z, np.float64)
    R = z.shape[0]
    return fwd_bwd(z, targets, float(dloss) / R if R > 0 else 0.0)["dz"]
