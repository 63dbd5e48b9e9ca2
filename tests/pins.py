"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an implementation namespace ``impl`` (the oracle module, or a
deliberately broken copy of it in the mutation tests) and returns an error
figure; ``PINS[op]`` lists (name, function, threshold).  A pin passes when
its error is at most its threshold.

What the pins compare against -- never a re-typed copy of the oracle's formula:
* central finite differences of the oracle's own forward (gradients);
* library routines: numpy matmul, math.fsum, scipy.special.expit / softmax /
  logsumexp, torch fp64 autograd of torch.mv, F.silu, torch.softmax,
  F.cross_entropy;
* a dense Jacobian built element by element (softmax);
* invariants (shapes, sums, bilinearity, shift invariance) and special cases;
* the weighted-sum page's worked tiling example (tests/golden).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def fd_grad(F, x, h_rel=1e-4):
    """Gradient of scalar F at x by the 4-point central stencil, per element."""
    x = np.array(x, np.float64, copy=True)
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for k in range(flat.size):
        h = h_rel * max(1.0, abs(flat[k]))
        x0 = flat[k]
        vals = []
        for step in (2, 1, -1, -2):
            flat[k] = x0 + step * h
            vals.append(F(x))
        flat[k] = x0
        gf[k] = (-vals[0] + 8 * vals[1] - 8 * vals[2] + vals[3]) / (12 * h)
    return g


def rel(a, b):
    """max |a - b| / max(|b|_inf, tiny) over all elements (inf-norm relative error)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.shape != b.shape:
        return np.inf
    if a.size == 0:
        return 0.0
    scale = max(float(np.max(np.abs(b))), 1e-300)
    return float(np.max(np.abs(a - b))) / scale


# ----------------------------------------------------------------------------- weighted sum

def ws_fwd_vs_matmul(impl):
    g = _rng(1)
    err = 0.0
    for n, d in [(1, 1), (7, 7), (7, 64), (33, 130)]:
        x = g.standard_normal((n, d))
        w = g.standard_normal(d)
        err = max(err, rel(impl.fwd(x, w), x @ w))
    return err


def ws_fwd_unit_weights_rowsum(impl):
    g = _rng(2)
    x = g.standard_normal((7, 19))
    ref = np.array([math.fsum(r) for r in x])
    return rel(impl.fwd(x, np.ones(19)), ref)


def ws_bwd_fd(impl):
    """grad_x and grad_w against finite differences of <dy, fwd(x, w)>; batch 1 and 7."""
    g = _rng(3)
    err = 0.0
    for n, d in [(1, 1), (1, 7), (7, 1), (7, 7), (7, 64)]:
        x = g.standard_normal((n, d))
        w = g.standard_normal(d)
        dy = g.standard_normal(n)
        gx, gw = impl.bwd(dy, x, w)
        fx = fd_grad(lambda xx: float(np.dot(dy, impl.fwd(xx, w))), x)
        fw = fd_grad(lambda ww: float(np.dot(dy, impl.fwd(x, ww))), w)
        err = max(err, rel(gx, fx), rel(gw, fw))
    return err


def ws_bwd_torch(impl):
    import torch

    g = _rng(4)
    x = g.standard_normal((7, 13))
    w = g.standard_normal(13)
    dy = g.standard_normal(7)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    torch.mv(xt, wt).backward(torch.tensor(dy))
    gx, gw = impl.bwd(dy, x, w)
    return max(rel(gx, xt.grad.numpy()), rel(gw, wt.grad.numpy()))


def ws_bilinear(impl):
    """<grad_w, w> = <grad_x, x> = <dy, y> (y is bilinear in x and w)."""
    g = _rng(5)
    x = g.standard_normal((9, 11))
    w = g.standard_normal(11)
    dy = g.standard_normal(9)
    gx, gw = impl.bwd(dy, x, w)
    s = float(np.dot(dy, impl.fwd(x, w)))
    scale = float(np.sum(np.abs(dy[:, None] * x * w[None, :])))
    return max(abs(float(np.dot(gw, w)) - s), abs(float(np.sum(gx * x)) - s)) / scale


def ws_accumulate(impl):
    """An existing grad_w is added into: bwd(old) - bwd(None) = old."""
    g = _rng(6)
    x = g.standard_normal((5, 4))
    w = g.standard_normal(4)
    dy = g.standard_normal(5)
    old = g.standard_normal(4)
    _, a = impl.bwd(dy, x, w, grad_w_old=old)
    _, b = impl.bwd(dy, x, w)
    return rel(a - b, old)


def ws_worked_tiling_case(impl):
    """The page's worked example: 100 rows, tiles of 32 rows, D = 64 -> partials [4, 64]."""
    gcase = golden("worked_tiling_case.json")
    n, d, bn = gcase["rows"], gcase["d"], gcase["block_n"]
    g = _rng(7)
    x = g.standard_normal((n, d))
    dy = g.standard_normal(n)
    w = g.standard_normal(d)
    P = impl.partials(x, dy, bn)
    if list(P.shape) != gcase["partial_shape"] or impl.n_tiles(n, bn) != gcase["n_row_tiles"]:
        return np.inf
    _, gw = impl.bwd(dy, x, w)
    if list(gw.shape) != gcase["grad_w_shape"]:
        return np.inf
    # the last tile holds the ragged rows 96..99 only
    lo, hi = gcase["last_tile_rows"]
    last = np.array([math.fsum(x[i, j] * dy[i] for i in range(lo, hi + 1)) for j in range(d)])
    return max(rel(P.sum(axis=0), gw), rel(P[-1], last))


def ws_interleaved_tiles(impl):
    """Rows dealt to tiles in blocks: 100 rows, blocks of 8, 3 tiles.  A one-hot
    dy at row 37 (block 4, so tile 1) puts x[37] into P[1] and zeros elsewhere;
    a dy that is 1 on rows 0..7 and 48..55 (blocks 0 and 6, both tile 0) puts
    the column sums of those rows into P[0]."""
    g = _rng(17)
    n, d = 100, 5
    x = g.standard_normal((n, d))
    dy = np.zeros(n)
    dy[37] = 1.0
    P = impl.partials(x, dy, 8, 3)
    if P.shape != (3, d):
        return np.inf
    err = max(rel(P[1], x[37]), float(np.max(np.abs(P[[0, 2]]))))
    dy = np.zeros(n)
    dy[0:8] = 1.0
    dy[48:56] = 1.0
    P = impl.partials(x, dy, 8, 3)
    want = np.array([math.fsum(list(x[0:8, j]) + list(x[48:56, j])) for j in range(d)])
    err = max(err, rel(P[0], want), float(np.max(np.abs(P[1:]))))
    # the ragged last block (rows 96..99, block 12) belongs to tile 0
    dy = np.zeros(n)
    dy[99] = 2.0
    P = impl.partials(x, dy, 8, 3)
    return max(err, rel(P[0], 2.0 * x[99]), float(np.max(np.abs(P[1:]))))


# ----------------------------------------------------------------------------- scaled SiLU

def silu_sigmoid_vs_expit(impl):
    from scipy.special import expit

    x = np.concatenate([np.linspace(-800, 800, 4001), np.linspace(-30, 30, 6001), [0.0]])
    return rel(impl.sigmoid(x), expit(x))


def silu_fwd_vs_torch(impl):
    import torch
    import torch.nn.functional as F

    g = _rng(8)
    x = g.standard_normal(1000) * 4
    w = 0.75
    ref = (w * F.silu(torch.tensor(x))).numpy()
    return rel(impl.fwd(x, w), ref)


def silu_bwd_fd(impl):
    g = _rng(9)
    err = 0.0
    for n in (1, 7, 64):
        x = g.standard_normal(n) * 2
        dy = g.standard_normal(n)
        w = 0.75
        dx, dw = impl.bwd(dy, x, w)
        fx = fd_grad(lambda xx: float(np.dot(dy, impl.fwd(xx, w))), x)
        fw = fd_grad(lambda ww: float(np.dot(dy, impl.fwd(x, float(ww[0])))), np.array([w]))
        err = max(err, rel(dx, fx), rel(np.array([dw]), fw))
    return err


def silu_bwd_torch(impl):
    import torch
    import torch.nn.functional as F

    g = _rng(10)
    x = g.standard_normal(257) * 3
    dy = g.standard_normal(257)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(0.75, dtype=torch.float64, requires_grad=True)
    (wt * F.silu(xt)).backward(torch.tensor(dy))
    dx, dw = impl.bwd(dy, x, 0.75)
    return max(rel(dx, xt.grad.numpy()), rel(np.array([dw]), np.array([wt.grad.item()])))


def silu_special_points(impl):
    """x = 0: y = 0 and dy/dx = w / 2; x -> +inf: y -> w x; x -> -inf: y -> 0."""
    w = 0.75
    y0 = impl.fwd(np.array([0.0]), w)[0]
    dx0, _ = impl.bwd(np.array([1.0]), np.array([0.0]), w)
    yb = impl.fwd(np.array([60.0, -60.0]), w)
    return max(abs(y0), abs(dx0[0] - w / 2), abs(yb[0] - w * 60.0) / 60.0, abs(yb[1]))


def silu_w_dw_invariant(impl):
    """y is linear in w, so w * dw = <dy, y>."""
    g = _rng(11)
    x = g.standard_normal(300) * 2
    dy = g.standard_normal(300)
    w = 0.75
    _, dw = impl.bwd(dy, x, w)
    y = impl.fwd(x, w)
    return abs(w * dw - float(np.dot(dy, y))) / float(np.sum(np.abs(dy * y)))


def silu_partials(impl):
    g = _rng(12)
    x = g.standard_normal(1000) * 2
    dy = g.standard_normal(1000)
    P = impl.partials(dy, x, 96)           # 11 tiles, the last one ragged (40 elements)
    _, dw = impl.bwd(dy, x, 0.75)
    _, dw_last = impl.bwd(dy[960:], x[960:], 0.75)
    if P.shape != (11,):
        return np.inf
    return max(abs(P.sum() - dw) / abs(dw), abs(P[-1] - dw_last) / max(abs(dw_last), 1e-300))


def silu_accumulate(impl):
    g = _rng(13)
    x = g.standard_normal(20)
    dy = g.standard_normal(20)
    _, a = impl.bwd(dy, x, 0.75, dw_old=2.5)
    _, b = impl.bwd(dy, x, 0.75)
    return abs((a - b) - 2.5) / 2.5


# ----------------------------------------------------------------------------- softmax

def softmax_fwd_vs_scipy(impl):
    from scipy.special import softmax

    g = _rng(14)
    x = g.standard_normal((9, 37)) * 3
    x[0, :] += 700.0   # would overflow exp without the max shift
    return rel(impl.fwd(x), softmax(x, axis=-1))


def softmax_fwd_invariants(impl):
    """Rows sum to 1; softmax(x + c) = softmax(x) for a per-row constant c; C = 1 gives 1."""
    g = _rng(15)
    x = g.standard_normal((7, 50)) * 3
    y = impl.fwd(x)
    c = g.standard_normal((7, 1)) * 10
    return max(float(np.max(np.abs(y.sum(-1) - 1))), rel(impl.fwd(x + c), y),
               float(np.max(np.abs(impl.fwd(np.zeros((3, 1))) - 1))))


def softmax_bwd_dense_jacobian(impl):
    """dx = J^T dy with J[i][j] = d y_i / d x_j = y_i (delta_ij - y_j), built entry by entry."""
    g = _rng(16)
    err = 0.0
    for C in (1, 2, 7, 16):
        x = g.standard_normal(C) * 2
        dy = g.standard_normal(C)
        y = impl.fwd(x[None, :])[0]
        J = [[y[i] * ((1.0 if i == j else 0.0) - y[j]) for j in range(C)] for i in range(C)]
        dx_ref = np.array([sum(J[i][j] * dy[i] for i in range(C)) for j in range(C)])
        dx = impl.bwd(dy[None, :], y[None, :])[0]
        err = max(err, float(np.max(np.abs(dx - dx_ref))) / max(1e-300, float(np.max(np.abs(dy)))))
    return err


def softmax_bwd_fd(impl):
    g = _rng(17)
    err = 0.0
    for R, C in [(1, 1), (1, 7), (7, 7), (2, 64)]:
        x = g.standard_normal((R, C)) * 2
        dy = g.standard_normal((R, C))
        dx = impl.bwd(dy, impl.fwd(x))
        fx = fd_grad(lambda xx: float(np.sum(dy * impl.fwd(xx))), x)
        err = max(err, float(np.max(np.abs(dx - fx))) / max(1e-300, float(np.max(np.abs(dy)))))
    return err


def softmax_bwd_torch(impl):
    import torch

    g = _rng(18)
    x = g.standard_normal((5, 33)) * 3
    dy = g.standard_normal((5, 33))
    xt = torch.tensor(x, requires_grad=True)
    torch.softmax(xt, dim=-1).backward(torch.tensor(dy))
    return rel(impl.bwd(dy, impl.fwd(x)), xt.grad.numpy())


def softmax_bwd_rows_sum_zero(impl):
    g = _rng(19)
    x = g.standard_normal((6, 40)) * 3
    dy = g.standard_normal((6, 40))
    dx = impl.bwd(dy, impl.fwd(x))
    return float(np.max(np.abs(dx.sum(-1)))) / float(np.max(np.abs(dy)))


def softmax_lse_vs_scipy(impl):
    from scipy.special import logsumexp

    g = _rng(21)
    x = g.standard_normal((8, 45)) * 3
    x[2] -= 900.0
    x[5] += 700.0
    return rel(impl.lse(x), logsumexp(x, axis=-1))


def softmax_bwd_from_x_torch(impl):
    """The rebuilt-y backward against torch fp64 autograd of softmax, batch 1 and 7."""
    import torch

    g = _rng(22)
    err = 0.0
    for R, C in [(1, 1), (1, 9), (7, 7), (7, 130)]:
        x = g.standard_normal((R, C)) * 3
        dy = g.standard_normal((R, C))
        xt = torch.tensor(x, requires_grad=True)
        torch.softmax(xt, dim=-1).backward(torch.tensor(dy))
        err = max(err, rel(impl.bwd_from_x(dy, x), xt.grad.numpy()))
    return err


def softmax_bwd_from_x_fd(impl):
    g = _rng(23)
    x = g.standard_normal((3, 11)) * 2
    dy = g.standard_normal((3, 11))
    fx = fd_grad(lambda xx: float(np.sum(dy * np.exp(xx - impl.lse(xx)[:, None]))), x)
    return rel(impl.bwd_from_x(dy, x), fx)


# ----------------------------------------------------------------------------- softmax-xent

def _xent_case(seed, R, C, sigma=2.0):
    g = _rng(seed)
    z = g.standard_normal((R, C)) * sigma
    t = g.integers(0, C, size=R)
    return z, t


def xent_vs_torch(impl):
    """loss and dz against torch's fp64 cross_entropy (mean) and its autograd."""
    import torch
    import torch.nn.functional as F

    err = 0.0
    for R, C in [(1, 1), (1, 2), (7, 7), (7, 64), (3, 1000)]:
        z, t = _xent_case(20 + R + C, R, C)
        zt = torch.tensor(z, requires_grad=True)
        loss = F.cross_entropy(zt, torch.tensor(t), reduction="mean")
        loss.backward()
        out = impl.fwd_bwd(z, t, 1.0 / R)
        err = max(err, abs(out["loss"] - loss.item()) / max(1.0, abs(loss.item())),
                  rel(out["dz"], zt.grad.numpy()))
    return err


def xent_stats_vs_scipy(impl):
    from scipy.special import logsumexp

    z, t = _xent_case(30, 7, 500)
    z[3] += 800.0
    out = impl.fwd_bwd(z, t, 1.0 / 7)
    return max(rel(out["row_lse"], logsumexp(z, axis=1)), rel(out["row_max"], z.max(axis=1)))


def xent_bwd_fd(impl):
    """dz against finite differences of the mean loss (grad_scale = 1 / R); batch 1 and 7."""
    err = 0.0
    for R, C in [(1, 1), (1, 7), (7, 2), (7, 7)]:
        z, t = _xent_case(40 + R * C, R, C)
        dz = impl.fwd_bwd(z, t, 1.0 / R)["dz"]
        fz = fd_grad(lambda zz: float(impl.fwd_bwd(zz, t, 1.0 / R)["loss"]), z)
        err = max(err, rel(dz, fz) if np.max(np.abs(fz)) > 0 else float(np.max(np.abs(dz))))
    return err


def xent_softmax_minus_onehot(impl):
    """dz / grad_scale = softmax(z) - e_t, with softmax from scipy."""
    from scipy.special import softmax

    z, t = _xent_case(50, 7, 300)
    scale = 2.0 ** -14
    dz = impl.fwd_bwd(z, t, scale)["dz"]
    ref = softmax(z, axis=1)
    ref[np.arange(7), t] -= 1.0
    return rel(dz / scale, ref)


def xent_special_cases(impl):
    """Uniform logits: loss = log C, dz = s (1/C - e_t); rows of dz sum to 0; shift invariance."""
    C, R = 37, 5
    t = np.array([0, 5, 36, 17, 2])
    out = impl.fwd_bwd(np.full((R, C), 1.25), t, 0.5)
    ref = np.full((R, C), 0.5 / C)
    ref[np.arange(R), t] -= 0.5
    e1 = max(abs(out["loss"] - math.log(C)) / math.log(C), rel(out["dz"], ref))
    z, t2 = _xent_case(60, 6, 90)
    a = impl.fwd_bwd(z, t2, 1.0)
    b = impl.fwd_bwd(z + 123.0, t2, 1.0)
    e2 = float(np.max(np.abs(a["dz"].sum(axis=1))))
    e3 = max(abs(a["loss"] - b["loss"]) / abs(a["loss"]), rel(b["dz"], a["dz"]))
    return max(e1, e2, e3)


def xent_invalid_targets(impl):
    """Reading for targets outside [0, C): NaN row loss, no one-hot term, counted."""
    z, _ = _xent_case(70, 4, 9)
    t = np.array([3, -1, 9, 0])
    out = impl.fwd_bwd(z, t, 1.0)
    from scipy.special import softmax

    p = softmax(z, axis=1)
    ok = (out["n_invalid"] == 2 and np.isnan(out["row_loss"][1]) and np.isnan(out["row_loss"][2])
          and np.isnan(out["loss"]) and np.all(np.isfinite(out["row_loss"][[0, 3]])))
    return max(rel(out["dz"][1], p[1]), rel(out["dz"][2], p[2])) if ok else np.inf


def xent_split_vs_torch(impl):
    """Split forward / backward against torch fp64 cross_entropy with an upstream
    gradient other than 1 (batch 1 and 7)."""
    import torch
    import torch.nn.functional as F

    err = 0.0
    for R, C in [(1, 1), (1, 5), (7, 7), (7, 300)]:
        z, t = _xent_case(80 + R + C, R, C)
        zt = torch.tensor(z, requires_grad=True)
        loss = F.cross_entropy(zt, torch.tensor(t), reduction="mean")
        loss.backward(torch.tensor(-2.5, dtype=torch.float64))
        f = impl.fwd(z, t)
        err = max(err, abs(f["loss"] - loss.item()) / max(1.0, abs(loss.item())),
                  rel(impl.bwd(z, t, -2.5), zt.grad.numpy()))
    return err


def xent_split_stats(impl):
    """Forward statistics of the split form against scipy (lse) and numpy (max, loss rows)."""
    from scipy.special import logsumexp

    z, t = _xent_case(90, 6, 77)
    z[1] -= 500.0
    f = impl.fwd(z, t)
    rows = np.arange(6)
    return max(rel(f["row_lse"], logsumexp(z, axis=1)), rel(f["row_max"], z.max(axis=1)),
               rel(f["row_loss"], logsumexp(z, axis=1) - z[rows, t]),
               0.0 if ("dz" not in f and f["n_invalid"] == 0) else np.inf)


# ----------------------------------------------------------------------------- norms

def _norm_case(seed, R, D, scale=2.0):
    g = _rng(seed)
    x = g.standard_normal((R, D)) * scale + g.standard_normal((R, 1))
    w = 1.0 + 0.3 * g.standard_normal(D)
    b = 0.2 * g.standard_normal(D)
    dy = g.standard_normal((R, D))
    return x, w, b, dy


def ln_fwd_vs_torch(impl):
    import torch
    import torch.nn.functional as F

    x, w, b, _ = _norm_case(110, 7, 65)
    y, mu, rstd = impl.layernorm_fwd(x, w, b, 1e-5)
    ref = F.layer_norm(torch.tensor(x), (65,), torch.tensor(w), torch.tensor(b), 1e-5).numpy()
    return max(rel(y, ref), rel(mu, x.mean(axis=1)), rel(rstd, 1.0 / np.sqrt(x.var(axis=1) + 1e-5)))


def ln_bwd_vs_torch(impl):
    """dx, dw, db against torch fp64 autograd of layer_norm, batch 1 and 7."""
    import torch
    import torch.nn.functional as F

    err = 0.0
    for R, D in [(1, 1), (1, 9), (7, 7), (7, 130)]:
        x, w, b, dy = _norm_case(111 + R + D, R, D)
        xt, wt, bt = (torch.tensor(a, requires_grad=True) for a in (x, w, b))
        F.layer_norm(xt, (D,), wt, bt, 1e-5).backward(torch.tensor(dy))
        dx, dw, db = impl.layernorm_bwd(dy, x, w, 1e-5)
        err = max(err, rel(dx, xt.grad.numpy()) if D > 1 else float(np.max(np.abs(dx))),
                  rel(dw, wt.grad.numpy()) if D > 1 else 0.0, rel(db, bt.grad.numpy()))
    return err


def ln_bwd_fd(impl):
    """Finite differences of sum(dy * y) with respect to x, w and b."""
    x, w, b, dy = _norm_case(112, 3, 6)
    dx, dw, db = impl.layernorm_bwd(dy, x, w, 1e-3)
    fx = fd_grad(lambda xx: float(np.sum(dy * impl.layernorm_fwd(xx, w, b, 1e-3)[0])), x)
    fw = fd_grad(lambda ww: float(np.sum(dy * impl.layernorm_fwd(x, ww, b, 1e-3)[0])), w)
    fb = fd_grad(lambda bb: float(np.sum(dy * impl.layernorm_fwd(x, w, bb, 1e-3)[0])), b)
    return max(rel(dx, fx), rel(dw, fw), rel(db, fb))


def ln_invariants(impl):
    """Rows of dx sum to 0 (shift invariance) and, with eps -> 0, dx is orthogonal
    to xhat (scale invariance); db = column sums of dy."""
    x, w, b, dy = _norm_case(113, 5, 40)
    dx, dw, db = impl.layernorm_bwd(dy, x, w, 1e-12)
    mu, rstd = impl.layernorm_stats(x, 1e-12)
    xhat = (x - mu[:, None]) * rstd[:, None]
    scale = float(np.max(np.abs(dx)))
    return max(float(np.max(np.abs(dx.sum(axis=1)))) / scale,
               float(np.max(np.abs((dx * xhat).sum(axis=1)))) / scale / 40,
               rel(db, np.array([math.fsum(dy[:, j]) for j in range(40)])))


def ln_accumulate(impl):
    x, w, b, dy = _norm_case(114, 4, 9)
    g = _rng(114)
    ow, ob = g.standard_normal(9), g.standard_normal(9)
    _, a1, a2 = impl.layernorm_bwd(dy, x, w, 1e-5, dw_old=ow, db_old=ob)
    _, b1, b2 = impl.layernorm_bwd(dy, x, w, 1e-5)
    return max(rel(a1 - b1, ow), rel(a2 - b2, ob))


def rms_fwd_vs_torch(impl):
    import torch
    import torch.nn.functional as F

    x, w, _, _ = _norm_case(115, 7, 65)
    y, rstd = impl.rmsnorm_fwd(x, w, 1e-6)
    ref = F.rms_norm(torch.tensor(x), (65,), torch.tensor(w), 1e-6).numpy()
    return max(rel(y, ref), rel(rstd, 1.0 / np.sqrt(np.mean(x * x, axis=1) + 1e-6)))


def rms_bwd_vs_torch(impl):
    import torch
    import torch.nn.functional as F

    err = 0.0
    for R, D in [(1, 1), (1, 9), (7, 7), (7, 130)]:
        x, w, _, dy = _norm_case(116 + R + D, R, D)
        xt, wt = torch.tensor(x, requires_grad=True), torch.tensor(w, requires_grad=True)
        F.rms_norm(xt, (D,), wt, 1e-6).backward(torch.tensor(dy))
        dx, dw = impl.rmsnorm_bwd(dy, x, w, 1e-6)
        # dx cancels (g - xhat c) almost exactly at D = 1: measure against |g rstd|
        scale = float(np.max(np.abs(dy * w / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + 1e-6))))
        err = max(err, float(np.max(np.abs(dx - xt.grad.numpy()))) / scale, rel(dw, wt.grad.numpy()))
    return err


def rms_bwd_fd(impl):
    x, w, _, dy = _norm_case(117, 3, 6)
    dx, dw = impl.rmsnorm_bwd(dy, x, w, 1e-3)
    fx = fd_grad(lambda xx: float(np.sum(dy * impl.rmsnorm_fwd(xx, w, 1e-3)[0])), x)
    fw = fd_grad(lambda ww: float(np.sum(dy * impl.rmsnorm_fwd(x, ww, 1e-3)[0])), w)
    return max(rel(dx, fx), rel(dw, fw))


def rms_scale_invariance(impl):
    """With eps -> 0, RMSNorm(a x) = RMSNorm(x) for a > 0, so dx . x = 0 per row."""
    x, w, _, dy = _norm_case(118, 5, 33)
    dx, _ = impl.rmsnorm_bwd(dy, x, w, 1e-14)
    return float(np.max(np.abs((dx * x).sum(axis=1)))) / float(np.max(np.abs(dx)) * np.max(np.abs(x)) * 33)


def rms_accumulate(impl):
    x, w, _, dy = _norm_case(119, 4, 9)
    ow = _rng(119).standard_normal(9)
    _, a = impl.rmsnorm_bwd(dy, x, w, 1e-6, dw_old=ow)
    _, b = impl.rmsnorm_bwd(dy, x, w, 1e-6)
    return rel(a - b, ow)


# ----------------------------------------------------------------------------- gather / scatter-add

def _gather_case(seed, M, V, D, dup=True):
    g = _rng(seed)
    x = g.standard_normal((V, D))
    idx = g.integers(0, max(1, V // 3) if dup else V, size=M) if dup else g.permutation(V)[:M]
    dy = g.standard_normal((M, D))
    return x, idx, dy


def gather_fwd_vs_take(impl):
    x, idx, _ = _gather_case(130, 50, 20, 7)
    return rel(impl.fwd(x, idx), np.take(x, idx, axis=0))


def gather_bwd_vs_add_at(impl):
    """numpy's unbuffered scatter-add, batch 1 and 7 and a longer case."""
    err = 0.0
    for M, V, D in [(1, 3, 4), (7, 5, 3), (200, 30, 9)]:
        x, idx, dy = _gather_case(131 + M, M, V, D)
        ref = np.zeros((V, D))
        np.add.at(ref, idx, dy)
        dx, n_inv = impl.bwd(dy, idx, V)
        err = max(err, rel(dx, ref) if np.any(ref) else float(np.max(np.abs(dx))), float(n_inv))
    return err


def gather_bwd_one_hot_matmul(impl):
    """dx = O^T dy with O[m, v] = [idx[m] = v], the Jacobian of the gather."""
    x, idx, dy = _gather_case(132, 40, 12, 5)
    O = np.zeros((40, 12))
    O[np.arange(40), idx] = 1.0
    return rel(impl.bwd(dy, idx, 12)[0], O.T @ dy)


def gather_bwd_fd(impl):
    x, idx, dy = _gather_case(133, 9, 6, 3)
    dx, _ = impl.bwd(dy, idx, 6)
    fx = fd_grad(lambda xx: float(np.sum(dy * impl.fwd(xx, idx))), x)
    return rel(dx, fx)


def gather_conservation(impl):
    """Every upstream row lands in exactly one table row: column sums agree, rows
    never selected stay zero; distinct indices reduce to a plain scatter."""
    x, idx, dy = _gather_case(134, 100, 40, 6)
    dx, _ = impl.bwd(dy, idx, 40)
    unused = np.setdiff1d(np.arange(40), idx)
    e1 = rel(dx.sum(axis=0), np.array([math.fsum(dy[:, j]) for j in range(6)]))
    e2 = float(np.max(np.abs(dx[unused]))) if unused.size else 0.0
    x, idx2, dy2 = _gather_case(135, 15, 40, 6, dup=False)
    dx2, _ = impl.bwd(dy2, idx2, 40)
    return max(e1, e2, rel(dx2[idx2], dy2))


def gather_invalid_and_order(impl):
    """A hand-worked case: idx = [3, 1, 3, 0, 1, 3, -1, 5], V = 5.  Rows 6 and 7
    are invalid (counted, no contribution, zero output row); the stable order by
    index is 0 (m = 3), 1 (m = 1, 4), 3 (m = 0, 2, 5), then the invalid m = 6, 7."""
    idx = np.array([3, 1, 3, 0, 1, 3, -1, 5])
    V, D = 5, 2
    dy = np.arange(16, dtype=np.float64).reshape(8, 2) + 1.0
    dx, n_inv = impl.bwd(dy, idx, V)
    want = np.zeros((V, D))
    want[0] = dy[3]
    want[1] = dy[1] + dy[4]
    want[3] = dy[0] + dy[2] + dy[5]
    order_ok = list(impl.sorted_order(idx, V)) == [3, 1, 4, 0, 2, 5, 6, 7]
    counts_ok = list(impl.counts(idx, V)) == [1, 2, 0, 3, 0]
    y = impl.fwd(np.ones((V, D)), idx)
    fwd_ok = bool(np.all(y[6:] == 0) and np.all(y[:6] == 1))
    ok = order_ok and counts_ok and fwd_ok and n_inv == 2
    return rel(dx, want) if ok else np.inf


def gather_accumulate(impl):
    x, idx, dy = _gather_case(136, 30, 10, 4)
    old = _rng(136).standard_normal((10, 4))
    a, _ = impl.bwd(dy, idx, 10, dx_old=old)
    b, _ = impl.bwd(dy, idx, 10)
    return rel(a - b, old)


PINS = {
    "weighted_sum": [
        ("fwd_vs_matmul", ws_fwd_vs_matmul, 1e-12),
        ("fwd_unit_weights_rowsum", ws_fwd_unit_weights_rowsum, 1e-13),
        ("bwd_finite_differences", ws_bwd_fd, 1e-9),
        ("bwd_vs_torch_autograd", ws_bwd_torch, 1e-13),
        ("bilinearity", ws_bilinear, 1e-13),
        ("accumulate", ws_accumulate, 1e-13),
        ("worked_tiling_case", ws_worked_tiling_case, 1e-12),
        ("interleaved_tiles", ws_interleaved_tiles, 1e-15),
    ],
    "scaled_silu": [
        ("sigmoid_vs_expit", silu_sigmoid_vs_expit, 1e-15),
        ("fwd_vs_torch_silu", silu_fwd_vs_torch, 1e-14),
        ("bwd_finite_differences", silu_bwd_fd, 1e-9),
        ("bwd_vs_torch_autograd", silu_bwd_torch, 1e-13),
        ("special_points", silu_special_points, 1e-14),
        ("w_dw_invariant", silu_w_dw_invariant, 1e-13),
        ("partials", silu_partials, 1e-12),
        ("accumulate", silu_accumulate, 1e-13),
    ],
    "softmax": [
        ("fwd_vs_scipy", softmax_fwd_vs_scipy, 1e-13),
        ("fwd_invariants", softmax_fwd_invariants, 1e-13),
        ("bwd_dense_jacobian", softmax_bwd_dense_jacobian, 1e-14),
        ("bwd_finite_differences", softmax_bwd_fd, 1e-9),
        ("bwd_vs_torch_autograd", softmax_bwd_torch, 1e-13),
        ("bwd_rows_sum_zero", softmax_bwd_rows_sum_zero, 1e-14),
        ("lse_vs_scipy", softmax_lse_vs_scipy, 1e-14),
        ("bwd_from_x_vs_torch", softmax_bwd_from_x_torch, 1e-13),
        ("bwd_from_x_finite_differences", softmax_bwd_from_x_fd, 1e-9),
    ],
    "softmax_xent": [
        ("vs_torch_cross_entropy", xent_vs_torch, 1e-13),
        ("stats_vs_scipy", xent_stats_vs_scipy, 1e-14),
        ("bwd_finite_differences", xent_bwd_fd, 1e-8),
        ("softmax_minus_onehot", xent_softmax_minus_onehot, 1e-13),
        ("special_cases", xent_special_cases, 1e-13),
        ("invalid_targets", xent_invalid_targets, 1e-13),
        ("split_vs_torch", xent_split_vs_torch, 1e-13),
        ("split_stats", xent_split_stats, 1e-14),
    ],
    "norms": [
        ("ln_fwd_vs_torch", ln_fwd_vs_torch, 1e-13),
        ("ln_bwd_vs_torch_autograd", ln_bwd_vs_torch, 1e-12),
        ("ln_bwd_finite_differences", ln_bwd_fd, 1e-8),
        ("ln_invariants", ln_invariants, 1e-10),
        ("ln_accumulate", ln_accumulate, 1e-13),
        ("rms_fwd_vs_torch", rms_fwd_vs_torch, 1e-13),
        ("rms_bwd_vs_torch_autograd", rms_bwd_vs_torch, 1e-12),
        ("rms_bwd_finite_differences", rms_bwd_fd, 1e-8),
        ("rms_scale_invariance", rms_scale_invariance, 1e-12),
        ("rms_accumulate", rms_accumulate, 1e-13),
    ],
    "gather": [
        ("fwd_vs_take", gather_fwd_vs_take, 0.0),
        ("bwd_vs_add_at", gather_bwd_vs_add_at, 1e-15),
        ("bwd_one_hot_matmul", gather_bwd_one_hot_matmul, 1e-14),
        ("bwd_finite_differences", gather_bwd_fd, 1e-9),
        ("conservation_and_distinct", gather_conservation, 1e-14),
        ("invalid_and_order", gather_invalid_and_order, 0.0),
        ("accumulate", gather_accumulate, 1e-14),
    ],
}
