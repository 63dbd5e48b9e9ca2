"""Row and tile counts past the per-launch limits: more than 2^20 rows (the
row ops launch in chunks of 2^20 rows) and more than 2^20 tiles (the
weighted-sum backward's reader workgroups loop over the tiles).  Narrow rows keep
the inputs small; every output element is compared with the oracle at the
bars of the per-op suites (both sides of each chunk boundary included)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, to_host
from oracle.compare import U32, exact, pointwise, reduced
from oracle.rounding import round_to, to_storage
from test_gpu_norms import _check, _stat_errors, bwd_bound, fwd_bound
from test_gpu_softmax_lse import _lse_S

pytestmark = pytest.mark.gpu
BIG = (1 << 20) + 3


def _sample(n, seed):
    """Every row (the name is kept for the call sites; seed is unused)."""
    return np.arange(n)


def test_weighted_sum_more_tiles_than_workgroups(gpu_lib):
    """One-row tiles over 2^20 + 3 rows: 2^20 + 3 tiles for 512 reader workgroups."""
    n, d = BIG, 2
    print(f"\n[weighted_sum tiles>2^20] n={n} d={d} rows_per_tile=1", flush=True)
    x = synth.normal((n, d), 1.0, "f32", 700, synth.STREAM_X)
    w = synth.normal((d,), 1.0, "f32", 700, synth.STREAM_W)
    dy = synth.normal((n,), 1.0, "f32", 700, synth.STREAM_DY)
    x64, w64, dy64 = synth.to_f64(x, "f32"), synth.to_f64(w, "f32"), synth.to_f64(dy, "f32")
    br, tiles = gpu_lib.vjp_weighted_sum_tiling(n, 1)
    assert (br, tiles) == (1, n)
    ws = torch.empty(gpu_lib.vjp_weighted_sum_bwd_workspace_size(n, d, 1) // 4, dtype=torch.float32,
                     device=DEV)
    dx, dw = gpu_lib.vjp_weighted_sum_bwd(synth.to_torch(dy, "f32", DEV),
                                          synth.to_torch(x, "f32", DEV).view(n, d),
                                          synth.to_torch(w, "f32", DEV), rows_per_tile=1, workspace=ws)
    gx, gw = oracle.weighted_sum.bwd(dy64, x64, w64)
    idx = _sample(n, 1)
    # one-row tiles: partial row t is x[t, :] dy[t]
    P_ref = oracle.weighted_sum.partials(x64[idx], dy64[idx], 1)
    reps = [exact(to_host(dx, "f32"), to_storage(round_to(gx, "f32"), "f32"), "f32", name="dx"),
            reduced(to_host(dw, "f32"), gw, name="dw"),
            pointwise(to_host(ws, "f32").reshape(n, d)[idx], P_ref, "f32", name="partials(all rows)")]
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


def test_softmax_and_xent_more_rows_than_a_launch(gpu_lib):
    rows, C = BIG, 3
    print(f"\n[softmax/xent rows>2^20] rows={rows} C={C} bf16", flush=True)
    x = synth.normal((rows, C), 2.0, "bf16", 701, synth.STREAM_X)
    x64 = synth.to_f64(x, "bf16")
    xd = synth.to_torch(x, "bf16", DEV).view(rows, C)
    idx = _sample(rows, 2)
    xs = x64[idx]
    y, lse = gpu_lib.vjp_softmax_fwd_lse(xd)
    reps = [pointwise(to_host(y, "bf16")[idx], oracle.softmax.fwd(xs), "bf16", name="y(all rows)"),
            pointwise(to_host(lse, "f32")[idx], oracle.softmax.lse(xs), "f32", S=_lse_S(xs),
                      name="lse(all rows)")]
    t = synth.targets(rows, C, 701)
    scale = 1.0 / rows
    out = gpu_lib.vjp_softmax_xent_fwd_bwd(xd, torch.from_numpy(t).to(DEV), grad_scale=scale)
    ref = oracle.softmax_xent.fwd_bwd(xs, t[idx], scale)
    p = np.exp(xs - ref["row_lse"][:, None])
    onehot = np.zeros_like(p)
    onehot[np.arange(len(idx)), t[idx]] = 1.0
    reps.append(pointwise(to_host(out["dlogits"], "bf16")[idx], ref["dz"], "bf16",
                          S=scale * (p + onehot), floor=16 * U32 * scale * onehot, name="dlogits(all rows)"))
    reps.append(reduced(to_host(out["loss"], "f32"),
                        np.array([oracle.softmax_xent.fwd(x64, t)["loss"]]), name="loss"))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


def test_rmsnorm_more_rows_than_a_launch(gpu_lib):
    rows, cols, eps = BIG, 4, 1e-6
    print(f"\n[rmsnorm rows>2^20] rows={rows} cols={cols} f32", flush=True)
    x = synth.normal((rows, cols), 1.0, "f32", 702, synth.STREAM_X)
    dy = synth.normal((rows, cols), 1.0, "f32", 702, synth.STREAM_DY)
    x64, dy64 = synth.to_f64(x, "f32"), synth.to_f64(dy, "f32")
    w64 = np.ones(cols)
    xd = synth.to_torch(x, "f32", DEV).view(rows, cols)
    wd = torch.ones(cols, device=DEV)
    y, rstd = gpu_lib.vjp_rmsnorm_fwd(xd, wd, eps)
    # the backward takes the oracle's rstd rounded to fp32, as the norm suite does
    rstd_ref = oracle.norms.rmsnorm_rstd(x64, eps)
    dx, dw = gpu_lib.vjp_rmsnorm_bwd(synth.to_torch(dy, "f32", DEV).view(rows, cols), xd, wd,
                                     torch.from_numpy(rstd_ref.astype(np.float32)).to(DEV), eps)
    idx = _sample(rows, 3)
    xs, dys = x64[idx], dy64[idx]
    y_ref, _ = oracle.norms.rmsnorm_fwd(xs, w64, eps)
    _, dr = _stat_errors(xs, 0.0, rstd_ref[idx, None], eps, True, saved=False)
    dx_ref, _ = oracle.norms.rmsnorm_bwd(dys, xs, w64, eps)
    _, dw_ref = oracle.norms.rmsnorm_bwd(dy64, x64, w64, eps)
    reps = [_check(to_host(y, "f32")[idx], y_ref, fwd_bound(xs, w64, 0.0, eps, True), "f32", "y(all rows)"),
            _check(to_host(dx, "f32")[idx], dx_ref, bwd_bound(dys, xs, w64, eps, True, True), "f32",
                   "dx(all rows)"),
            pointwise(to_host(rstd, "f32")[idx], rstd_ref[idx], "f32", S=2 * dr[:, 0] * rstd_ref[idx] / 1e-5,
                      name="rstd(all rows)"),
            reduced(to_host(dw, "f32"), dw_ref, name="dw")]
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]
