"""LayerNorm and RMSNorm over the last dimension and their VJPs, in fp64 --
test infrastructure.

Source: "Backprop for kernel writers", the LayerNorm passage after 04 "The
duality" (LayerNorm couples every element of a row through its mean and
variance, yet its backward collapses to two row scalars; the parameter
gradients reduce over the batch axis) and section 07 (LayerNorm backward:
two accumulators plus a batch-axis parameter reduction).  "Backward in
Triton -- autograd.Function and the backward grid", sections "Save vs
recompute" (the rstd is a one-scalar-per-row statistic) and "The backward
grid is not the forward grid" (RMSNorm's dw sums a length-d partial from
every row).

The pages give no formulas (they are lost in extraction); the definitions
below are the standard ones, written from the forward by differentiation:

LayerNorm, row x of D values, eps > 0:
  mu = (1/D) sum_j x_j,  var = (1/D) sum_j (x_j - mu)^2,  rstd = 1/sqrt(var + eps)
  xhat_j = (x_j - mu) rstd,   y_j = xhat_j w_j + b_j
  g_j = dy_j w_j
  dx_j = rstd (g_j - (1/D) sum_k g_k - xhat_j (1/D) sum_k g_k xhat_k)
  dw_j = sum over rows of dy_j xhat_j,   db_j = sum over rows of dy_j
RMSNorm:
  rstd = 1/sqrt((1/D) sum_j x_j^2 + eps),  xhat_j = x_j rstd,  y_j = xhat_j w_j
  dx_j = rstd (g_j - xhat_j (1/D) sum_k g_k xhat_k),   dw_j = sum over rows of dy_j xhat_j

The backward here is that closed form; the pins check it against torch's
fp64 autograd of its own layer_norm / rms_norm and finite differences of
:func:`layernorm_fwd` / :func:`rmsnorm_fwd`.
"""
from __future__ import annotations

import numpy as np


def layernorm_stats(x, eps):
    x = np.asarray(x, np.float64)
    mu = np.mean(x, axis=-1)
    var = np.mean((x - mu[..., None]) ** 2, axis=-1)
    return mu, 1.0 / np.sqrt(var + eps)


def layernorm_fwd(x, w, b, eps):
    """Returns (y, mean, rstd)."""
    x = np.asarray(x, np.float64)
    mu, rstd = layernorm_stats(x, eps)
    xhat = (x - mu[..., None]) * rstd[..., None]
    return xhat * np.asarray(w, np.float64) + np.asarray(b, np.float64), mu, rstd


def layernorm_bwd(dy, x, w, eps, dw_old=None, db_old=None):
    """Returns (dx, dw, db); dw / db are added into dw_old / db_old when given."""
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    mu, rstd = layernorm_stats(x, eps)
    xhat = (x - mu[..., None]) * rstd[..., None]
    g = dy * w
    a = np.mean(g, axis=-1, keepdims=True)
    c = np.mean(g * xhat, axis=-1, keepdims=True)
    dx = rstd[..., None] * (g - a - xhat * c)
    dw = np.sum((dy * xhat).reshape(-1, x.shape[-1]), axis=0)
    db = np.sum(dy.reshape(-1, x.shape[-1]), axis=0)
    if dw_old is not None:
        dw = np.asarray(dw_old, np.float64) + dw
    if db_old is not None:
        db = np.asarray(db_old, np.float64) + db
    return dx, dw, db


def rmsnorm_rstd(x, eps):
    x = np.asarray(x, np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)


def rmsnorm_fwd(x, w, eps):
    """Returns (y, rstd)."""
    x = np.asarray(x, np.float64)
    rstd = rmsnorm_rstd(x, eps)
    return x * rstd[..., None] * np.asarray(w, np.float64), rstd


def rmsnorm_bwd(dy, x, w, eps, dw_old=None):
    """Returns (dx, dw); dw is added into dw_old when given."""
    dy = np.asarray(dy, np.float64)
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    rstd = rmsnorm_rstd(x, eps)
    xhat = x * rstd[..., None]
    g = dy * w
    c = np.mean(g * xhat, axis=-1, keepdims=True)
    dx = rstd[..., None] * (g - xhat * c)
    dw = np.sum((dy * xhat).reshape(-1, x.shape[-1]), axis=0)
    if dw_old is not None:
        dw = np.asarray(dw_old, np.float64) + dw
    return dx, dw
