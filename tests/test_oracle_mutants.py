"""Planted mistakes in copies of the oracle must each fail at least one pin (no GPU).

This shows the pins are strong enough: a dropped term, a wrong sign, a
wrong index or a transposed operand anywhere in the oracle is caught.
Mutants are built here, on the CPU, from the oracle's own functions; the
oracle itself is never modified.
"""
import types

import numpy as np
import pytest

import oracle
from pins import PINS


def _ns(mod, **over):
    d = {k: getattr(mod, k) for k in dir(mod) if not k.startswith("_")}
    d.update(over)
    return types.SimpleNamespace(**d)


ws, silu, sm, xe = oracle.weighted_sum, oracle.scaled_silu, oracle.softmax, oracle.softmax_xent
nm = oracle.norms
ga = oracle.gather


def _ws_bwd_no_batch_reduction(dy, x, w, grad_w_old=None):
    gx, _ = ws.bwd(dy, x, w, grad_w_old)
    return gx, x[0] * dy[0]                       # correct at batch 1 only


def _ws_bwd_transposed(dy, x, w, grad_w_old=None):
    gx, gw = ws.bwd(dy, x, w, grad_w_old)
    return gx, np.sum(x * dy[:, None], axis=1)[: w.size] if x.shape[0] >= w.size else gw * 0


def _ws_bwd_overwrites(dy, x, w, grad_w_old=None):
    return ws.bwd(dy, x, w, None)                  # ignores the existing gradient


def _ws_partials_off_by_one(x, dy, block_rows, tiles=None):
    P = ws.partials(x, dy, block_rows, tiles)
    if tiles is None:
        P[-1] = np.sum(x[(P.shape[0] - 1) * block_rows + 1:] * dy[(P.shape[0] - 1) * block_rows + 1:, None], axis=0)
    return P


def _ws_partials_grouped(x, dy, block_rows, tiles=None):
    """Deals consecutive runs of blocks to a tile instead of round-robin."""
    n = x.shape[0]
    nb = ws.n_tiles(n, block_rows)
    T = nb if tiles is None else tiles
    per = -(-nb // T)
    P = np.zeros((T, x.shape[1]))
    for b in range(nb):
        lo, hi = b * block_rows, min((b + 1) * block_rows, n)
        P[b // per] += np.sum(x[lo:hi] * dy[lo:hi, None], axis=0)
    return P


def _silu_bwd_missing_term(dy, x, w, dw_old=None):
    s = silu.sigmoid(x)
    dx = dy * w * s                               # drops the x s (1 - s) term
    return dx, silu.bwd(dy, x, w, dw_old)[1]


def _silu_bwd_sign(dy, x, w, dw_old=None):
    s = silu.sigmoid(x)
    dx = dy * w * (s - x * s * (1 - s))
    return dx, silu.bwd(dy, x, w, dw_old)[1]


def _silu_dw_without_x(dy, x, w, dw_old=None):
    dx, _ = silu.bwd(dy, x, w, None)
    dw = float(np.sum(dy * silu.sigmoid(x)))
    return dx, dw if dw_old is None else dw + dw_old


def _silu_sigmoid_sign(x):
    return 1.0 / (1.0 + np.exp(np.clip(x, -700, 700)))


def _sm_bwd_sign(dy, y):
    return y * (dy + np.sum(dy * y, axis=-1, keepdims=True))


def _sm_bwd_wrong_axis(dy, y):
    return y * (dy - np.sum(dy * y, axis=0, keepdims=True))


def _sm_fwd_no_normalise(x):
    return np.exp(x - np.max(x, axis=-1, keepdims=True))


def _xent_no_onehot(z, t, grad_scale):
    out = xe.fwd_bwd(z, t, grad_scale)
    from scipy.special import softmax

    out["dz"] = grad_scale * softmax(z, axis=1)
    return out


def _xent_sum_not_mean(z, t, grad_scale):
    out = xe.fwd_bwd(z, t, grad_scale)
    out["loss"] = float(np.sum(out["row_loss"]))
    return out


def _xent_lse_without_max(z, t, grad_scale):
    out = xe.fwd_bwd(z, t, grad_scale)
    with np.errstate(over="ignore"):
        out["row_lse"] = np.log(np.sum(np.exp(z), axis=1)) - 0.0 * out["row_max"]
    out["row_lse"] = out["row_lse"] + (out["row_max"] > 100) * 1.0
    return out


def _sm_lse_no_max(x):
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore", divide="ignore"):
        return np.log(np.sum(np.exp(x), axis=-1))


def _sm_bwd_from_x_unnormalised(dy, x):
    e = np.exp(np.asarray(x) - np.max(x, axis=-1, keepdims=True))
    return sm.bwd(dy, e)


def _xent_bwd_sum_not_mean(z, t, dloss):
    return xe.fwd_bwd(z, t, float(dloss))["dz"]


def _xent_bwd_ignores_dloss(z, t, dloss):
    return xe.bwd(z, t, 1.0)


def _ln_bwd_no_mean_term(dy, x, w, eps, dw_old=None, db_old=None):
    dx, dw, db = nm.layernorm_bwd(dy, x, w, eps, dw_old, db_old)
    g = np.asarray(dy) * np.asarray(w)
    _, rstd = nm.layernorm_stats(x, eps)
    return dx + rstd[:, None] * np.mean(g, axis=-1, keepdims=True), dw, db


def _ln_bwd_dw_without_xhat(dy, x, w, eps, dw_old=None, db_old=None):
    dx, _, db = nm.layernorm_bwd(dy, x, w, eps, dw_old, db_old)
    return dx, np.sum(np.asarray(dy) * np.asarray(x), axis=0), db


def _ln_unbiased_var(x, eps):
    x = np.asarray(x, np.float64)
    return np.mean(x, axis=-1), 1.0 / np.sqrt(np.var(x, axis=-1, ddof=1) + eps)


def _ln_fwd_unbiased(x, w, b, eps):
    mu, rstd = _ln_unbiased_var(x, eps)
    return (np.asarray(x) - mu[:, None]) * rstd[:, None] * w + b, mu, rstd


def _rms_bwd_no_projection(dy, x, w, eps, dw_old=None):
    rstd = nm.rmsnorm_rstd(x, eps)
    dx = rstd[:, None] * np.asarray(dy) * np.asarray(w)
    return dx, nm.rmsnorm_bwd(dy, x, w, eps, dw_old)[1]


def _rms_bwd_dw_per_row(dy, x, w, eps, dw_old=None):
    dx, _ = nm.rmsnorm_bwd(dy, x, w, eps, dw_old)
    xhat = np.asarray(x) * nm.rmsnorm_rstd(x, eps)[:, None]
    return dx, (np.asarray(dy) * xhat)[0]


def _ga_plain_scatter(dy, idx, V, dx_old=None):
    dy = np.asarray(dy, np.float64)
    idx = np.asarray(idx)
    dx = np.zeros((V, dy.shape[1])) if dx_old is None else np.array(dx_old, np.float64)
    ok = (idx >= 0) & (idx < V)
    dx[idx[ok]] = dy[ok]                          # last write wins: duplicates dropped
    return dx, int(np.count_nonzero(~ok))


def _ga_order_descending_ties(idx, V):
    idx = np.asarray(idx, np.int64)
    key = np.where(ga.valid_mask(idx, V), idx, V)
    return np.lexsort((-np.arange(idx.size), key))


def _ga_fwd_wraps_invalid(x, idx):
    x = np.asarray(x, np.float64)
    return x[np.asarray(idx) % x.shape[0]]


MUTANTS = [
    ("weighted_sum", "bwd_no_batch_reduction", _ns(ws, bwd=_ws_bwd_no_batch_reduction)),
    ("weighted_sum", "bwd_transposed_reduction", _ns(ws, bwd=_ws_bwd_transposed)),
    ("weighted_sum", "bwd_overwrites_grad", _ns(ws, bwd=_ws_bwd_overwrites)),
    ("weighted_sum", "fwd_sign", _ns(ws, fwd=lambda x, w: -ws.fwd(x, w))),
    ("weighted_sum", "partials_off_by_one", _ns(ws, partials=_ws_partials_off_by_one)),
    ("weighted_sum", "partials_grouped_blocks", _ns(ws, partials=_ws_partials_grouped)),
    ("scaled_silu", "bwd_missing_term", _ns(silu, bwd=_silu_bwd_missing_term)),
    ("scaled_silu", "bwd_sign", _ns(silu, bwd=_silu_bwd_sign)),
    ("scaled_silu", "dw_without_x", _ns(silu, bwd=_silu_dw_without_x)),
    ("scaled_silu", "sigmoid_sign", _ns(silu, sigmoid=_silu_sigmoid_sign)),
    ("softmax", "bwd_sign", _ns(sm, bwd=_sm_bwd_sign)),
    ("softmax", "bwd_wrong_axis", _ns(sm, bwd=_sm_bwd_wrong_axis)),
    ("softmax", "fwd_not_normalised", _ns(sm, fwd=_sm_fwd_no_normalise)),
    ("softmax_xent", "no_onehot", _ns(xe, fwd_bwd=_xent_no_onehot)),
    ("softmax_xent", "sum_not_mean", _ns(xe, fwd_bwd=_xent_sum_not_mean)),
    ("softmax_xent", "lse_wrong", _ns(xe, fwd_bwd=_xent_lse_without_max)),
    ("softmax", "lse_without_max", _ns(sm, lse=_sm_lse_no_max)),
    ("softmax", "bwd_from_x_unnormalised", _ns(sm, bwd_from_x=_sm_bwd_from_x_unnormalised)),
    ("softmax_xent", "split_bwd_sum_not_mean", _ns(xe, bwd=_xent_bwd_sum_not_mean)),
    ("softmax_xent", "split_bwd_ignores_dloss", _ns(xe, bwd=_xent_bwd_ignores_dloss)),
    ("norms", "ln_bwd_no_mean_term", _ns(nm, layernorm_bwd=_ln_bwd_no_mean_term)),
    ("norms", "ln_bwd_dw_without_xhat", _ns(nm, layernorm_bwd=_ln_bwd_dw_without_xhat)),
    ("norms", "ln_unbiased_variance", _ns(nm, layernorm_fwd=_ln_fwd_unbiased, layernorm_stats=_ln_unbiased_var)),
    ("norms", "rms_bwd_no_projection", _ns(nm, rmsnorm_bwd=_rms_bwd_no_projection)),
    ("norms", "rms_bwd_dw_one_row", _ns(nm, rmsnorm_bwd=_rms_bwd_dw_per_row)),
    ("gather", "bwd_plain_scatter", _ns(ga, bwd=_ga_plain_scatter)),
    ("gather", "order_descending_ties", _ns(ga, sorted_order=_ga_order_descending_ties)),
    ("gather", "fwd_wraps_invalid", _ns(ga, fwd=_ga_fwd_wraps_invalid)),
]


@pytest.mark.parametrize("op,name,impl", MUTANTS, ids=[f"{m[0]}-{m[1]}" for m in MUTANTS])
def test_mutant_is_caught(op, name, impl):
    failed = []
    for pin_name, fn, thr in PINS[op]:
        try:
            with np.errstate(all="ignore"):
                err = fn(impl)
        except Exception:  # a crash also counts as caught
            err = np.inf
        if not (np.isfinite(err) and err <= thr):
            failed.append(pin_name)
    assert failed, f"planted mistake {op}/{name} passed every pin"
