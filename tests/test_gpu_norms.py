"""LayerNorm and RMSNorm forward / backward on the GPU vs the CPU oracle
(calls the C ABI).

Tolerances are bounds derived from the fp32 arithmetic of the kernels, with
a factor 2 margin (u = 2^-24; H = 40 bounds the depth of every fp32 row sum:
at most 16 sequential terms per lane, a 6-level wave tree and up to 16 waves
added in order):
  mean:  |d mu| <= H u mean|x| + 3 u |mu|          (saved fp32 input: u |mu|)
  rstd:  relative d r <= ((H + 4) u var + d mu^2) / (2 (var + eps)) + 2 u
                                                   (saved fp32 input: u)
  y:     |w| rstd (d mu + u |x - mu|) + |xhat w| (d r + u) + u |y|
  dx:    rstd d e + |dx| (d r + u), with e = g - a - xhat c and
         d e = u |g| + d a + |xhat| d c + |c| d xhat + 3 u (|g| + |a| + |xhat c|),
         d a = (H + 2) u mean|g|, d c = (H + 2) u mean|g xhat| + mean(|g| d xhat),
         d xhat = rstd (d mu + u |x - mu|) + |xhat| (d r + u)
fp32 outputs must lie within max(1e-5 |o|, bound); 16-bit outputs within 2 ulp
of the oracle rounded to the dtype or within 2 ulp(o) + bound.  dw and db:
||g - o||_2 <= 1e-4 ||o||_2.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, Guarded, chunked, empty_padded, padded, pick_rows, to_dev, to_host
from oracle.compare import U32 as U, combine, pointwise, reduced

pytestmark = pytest.mark.gpu
nm = oracle.norms
H = 40


def _stats64(x, eps, rms):
    if rms:
        return np.zeros((x.shape[0], 1)), nm.rmsnorm_rstd(x, eps)[:, None]
    mu, rstd = nm.layernorm_stats(x, eps)
    return mu[:, None], rstd[:, None]


def _stat_errors(x, mu, rstd, eps, rms, saved):
    var = 1.0 / rstd ** 2 - eps
    if saved:
        return U * np.abs(mu), np.full_like(rstd, U)
    dmu = 0.0 if rms else H * U * np.mean(np.abs(x), axis=1, keepdims=True) + 3 * U * np.abs(mu)
    dr = ((H + 4) * U * var + dmu ** 2) / (2 * (var + eps)) + 2 * U
    return dmu, dr


def fwd_bound(x, w, b, eps, rms):
    mu, rstd = _stats64(x, eps, rms)
    dmu, dr = _stat_errors(x, mu, rstd, eps, rms, saved=False)
    xh = (x - mu) * rstd
    y = xh * w + (0.0 if rms else b)
    return 2 * (np.abs(w) * rstd * (dmu + U * np.abs(x - mu)) + np.abs(xh * w) * (dr + U) + U * np.abs(y))


def bwd_bound(dy, x, w, eps, rms, saved):
    mu, rstd = _stats64(x, eps, rms)
    dmu, dr = _stat_errors(x, mu, rstd, eps, rms, saved)
    xh = (x - mu) * rstd
    g = dy * w
    dxh = rstd * (dmu + U * np.abs(x - mu)) + np.abs(xh) * (dr + U)
    a = 0.0 if rms else np.mean(g, axis=1, keepdims=True)
    da = 0.0 if rms else (H + 2) * U * np.mean(np.abs(g), axis=1, keepdims=True)
    c = np.mean(g * xh, axis=1, keepdims=True)
    dc = (H + 2) * U * np.mean(np.abs(g * xh), axis=1, keepdims=True) + np.mean(np.abs(g) * dxh, axis=1, keepdims=True)
    de = U * np.abs(g) + da + np.abs(xh) * dc + np.abs(c) * dxh + 3 * U * (np.abs(g) + np.abs(a) + np.abs(xh * c))
    dx = rstd * (g - a - xh * c)
    return 2 * (rstd * de + np.abs(dx) * (dr + U))


def _check(got, ref, bound, act, name):
    if act == "f32":
        return pointwise(got, ref, act, S=bound / 1e-5, name=name)
    return pointwise(got, ref, act, floor=bound, name=name)


def _inputs(rows, cols, act, wdt, seed, shift=0.0):
    x = synth.normal((rows, cols), 1.0, act, seed, synth.STREAM_X)
    if shift:
        x = synth.f32_to_storage(synth.to_f64(x, act).astype(np.float32) + np.float32(shift), act)
    g = np.random.default_rng(seed)
    w = synth.f32_to_storage((1.0 + 0.1 * g.standard_normal(cols)).astype(np.float32), wdt)
    b = synth.f32_to_storage((0.1 * g.standard_normal(cols)).astype(np.float32), wdt)
    dy = synth.normal((rows, cols), 1.0, act, seed, synth.STREAM_DY)
    return x, w, b, dy


def _param_dev(a, dtype, offset):
    """A device copy of a parameter vector starting `offset` elements into its buffer."""
    buf = torch.zeros(a.size + offset, dtype=synth.torch_dtype(dtype), device=DEV)
    buf[offset:] = to_dev(a, dtype)
    return buf[offset:]


def run_case(rwb, kind, rows, cols, act, wdt, seed, ld=None, offset=0, saved=True,
             accumulate=False, eps=None, shift=0.0, param_offset=0, ws_offset=0):
    rms = kind == "rms"
    eps = (1e-6 if rms else 1e-5) if eps is None else eps
    print(f"\n[{kind}] rows={rows} cols={cols} act={act} w={wdt} ld={ld} off={offset} "
          f"saved={saved} acc={accumulate} shift={shift}", flush=True)
    x, w, b, dy = _inputs(rows, cols, act, wdt, seed, shift)
    x64, w64, b64, dy64 = (synth.to_f64(x, act), synth.to_f64(w, wdt), synth.to_f64(b, wdt),
                           synth.to_f64(dy, act))
    xd, dyd = padded(x, act, ld, offset), padded(dy, act, ld, offset)
    wd, bd = _param_dev(w, wdt, param_offset), _param_dev(b, wdt, param_offset)
    y, _ = empty_padded(rows, cols, act, ld, offset)
    mean_g, rstd_g = Guarded(rows, torch.float32), Guarded(rows, torch.float32)
    if rms:
        rwb.vjp_rmsnorm_fwd(xd, wd, eps, y=y, row_rstd=rstd_g.t)
        y_ref, rstd_ref = nm.rmsnorm_fwd(x64, w64, eps)
        mu_ref = np.zeros(rows)
    else:
        rwb.vjp_layernorm_fwd(xd, wd, bd, eps, y=y, row_mean=mean_g.t, row_rstd=rstd_g.t)
        y_ref, mu_ref, rstd_ref = nm.layernorm_fwd(x64, w64, b64, eps)
    torch.cuda.synchronize()
    assert mean_g.intact() and rstd_g.intact()
    reps = [_check(to_host(y, act), y_ref, fwd_bound(x64, w64, b64, eps, rms), act, "y")]
    _, dr = _stat_errors(x64, mu_ref[:, None], rstd_ref[:, None], eps, rms, saved=False)
    reps.append(pointwise(to_host(rstd_g.t, "f32"), rstd_ref, "f32",
                          S=2 * dr[:, 0] * rstd_ref / 1e-5, name="row_rstd"))
    if not rms:
        dmu, _ = _stat_errors(x64, mu_ref[:, None], rstd_ref[:, None], eps, rms, saved=False)
        reps.append(pointwise(to_host(mean_g.t, "f32"), mu_ref, "f32", S=2 * dmu[:, 0] / 1e-5,
                              name="row_mean"))

    # backward: the oracle's statistics as fp32 inputs, or none (recomputed)
    g = np.random.default_rng(seed + 1)
    old_w = g.standard_normal(cols).astype(np.float32)
    old_b = g.standard_normal(cols).astype(np.float32)
    dwg, dbg = Guarded(cols, torch.float32), Guarded(cols, torch.float32)
    if accumulate:
        dwg.t.copy_(torch.from_numpy(old_w))
        dbg.t.copy_(torch.from_numpy(old_b))
    mu_in = torch.from_numpy(mu_ref.astype(np.float32)).to(DEV) if saved else None
    rstd_in = torch.from_numpy(rstd_ref.astype(np.float32)).to(DEV) if saved else None
    dx, _ = empty_padded(rows, cols, act, ld, offset)
    need = (rwb.vjp_rmsnorm_bwd_workspace_size if rms else rwb.vjp_layernorm_bwd_workspace_size)(rows, cols)
    wsg = Guarded(max(need // 4, 1) + ws_offset, torch.float32)
    ws = wsg.t[ws_offset:]                 # ws_offset = 1: 4-byte but not 16-byte aligned
    if rms:
        rwb.vjp_rmsnorm_bwd(dyd, xd, wd, rstd_in, eps, dx=dx, dw=dwg.t, accumulate=accumulate,
                            workspace=ws)
        dx_ref, dw_ref = nm.rmsnorm_bwd(dy64, x64, w64, eps, dw_old=old_w if accumulate else None)
    else:
        rwb.vjp_layernorm_bwd(dyd, xd, wd, mu_in, rstd_in, eps, dx=dx, dw=dwg.t, db=dbg.t,
                              accumulate=accumulate, workspace=ws)
        dx_ref, dw_ref, db_ref = nm.layernorm_bwd(dy64, x64, w64, eps,
                                                  dw_old=old_w if accumulate else None,
                                                  db_old=old_b if accumulate else None)
    torch.cuda.synchronize()
    assert dwg.intact() and dbg.intact() and wsg.intact(), "write outside an output"
    reps.append(_check(to_host(dx, act), dx_ref, bwd_bound(dy64, x64, w64, eps, rms, saved), act, "dx"))
    if rows > 0:
        reps.append(reduced(to_host(dwg.t, "f32"), dw_ref, name="dw"))
        if not rms:
            reps.append(reduced(to_host(dbg.t, "f32"), db_ref, name="db"))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


SHAPES = [(1, 1), (7, 7), (33, 100), (7, 512), (7, 513), (5, 4096), (3, 4097), (2, 16384),
          (1500, 64), (2049, 300)]
DTYPES = [("bf16", "bf16"), ("f16", "f16"), ("f32", "f32"), ("bf16", "f32"), ("f32", "bf16")]


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("rows,cols", SHAPES)
@pytest.mark.parametrize("act,wdt", DTYPES)
def test_shapes_dtypes(gpu_lib, kind, rows, cols, act, wdt):
    run_case(gpu_lib, kind, rows, cols, act, wdt, seed=400 + rows + cols)


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("rows,cols", [(7, 64), (1500, 300), (4, 9000)])
def test_recomputed_stats_and_accumulate(gpu_lib, kind, rows, cols):
    run_case(gpu_lib, kind, rows, cols, "bf16", "bf16", seed=410 + cols, saved=False, accumulate=True)


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("cols", [7, 4096, 12000])
@pytest.mark.parametrize("layout", ["padded_ld", "unaligned"])
def test_layouts(gpu_lib, kind, cols, layout):
    ld, off = (cols + 8, 0) if layout == "padded_ld" else (cols + 1, 1)
    run_case(gpu_lib, kind, 5, cols, "bf16", "bf16", seed=420 + cols, ld=ld, offset=off)


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("act, wdt, off", [("bf16", "bf16", 1), ("bf16", "f32", 1),
                                           ("bf16", "bf16", 4), ("bf16", "f32", 2),
                                           ("f32", "bf16", 1), ("f32", "f16", 2)])
def test_unaligned_parameters(gpu_lib, kind, act, wdt, off):
    """w and b `off` elements into their buffers (2 to 8 bytes past a 16-byte
    boundary): element-wise parameter loads in both passes, same values."""
    run_case(gpu_lib, kind, 9, 1000, act, wdt, seed=425, param_offset=off)


def _all_outputs(rwb, kind, xd, dyd, wd, bd):
    """y, the statistics, dx, dw (and db) of one forward and backward, as bits."""
    rows, cols = xd.shape
    y, dx = torch.empty_like(xd), torch.empty_like(xd)
    dw, db = torch.empty(cols, device=DEV), torch.empty(cols, device=DEV)
    if kind == "rms":
        _, rstd = rwb.vjp_rmsnorm_fwd(xd, wd, y=y)
        rwb.vjp_rmsnorm_bwd(dyd, xd, wd, rstd, dx=dx, dw=dw)
        outs = [y, rstd, dx, dw]
    else:
        _, mean, rstd = rwb.vjp_layernorm_fwd(xd, wd, bd, y=y)
        rwb.vjp_layernorm_bwd(dyd, xd, wd, mean, rstd, dx=dx, dw=dw, db=db)
        outs = [y, mean, rstd, dx, dw, db]
    torch.cuda.synchronize()
    return [o.cpu().view(torch.int16 if o.element_size() == 2 else torch.int32) for o in outs]


@pytest.mark.parametrize("kind", ["ln", "rms"])
@pytest.mark.parametrize("act, wdt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "bf16"),
                                      ("f16", "f16")])
@pytest.mark.parametrize("cols", [4096, 1000])
def test_parameter_loads_same_bits(gpu_lib, kind, act, wdt, cols):
    """w and b at a 16-byte boundary (loaded as vectors) and one element past
    it (loaded element by element) give the same bits in every output of the
    forward and the backward: both paths widen the same values to fp32."""
    rows = 300
    print(f"\n[{kind} parameter loads] rows={rows} cols={cols} act={act} w={wdt}", flush=True)
    x, w, b, dy = _inputs(rows, cols, act, wdt, 440 + cols)
    xd, dyd = padded(x, act), padded(dy, act)
    ref = _all_outputs(gpu_lib, kind, xd, dyd, _param_dev(w, wdt, 0), _param_dev(b, wdt, 0))
    got = _all_outputs(gpu_lib, kind, xd, dyd, _param_dev(w, wdt, 1), _param_dev(b, wdt, 1))
    same = [torch.equal(a, c) for a, c in zip(ref, got)]
    print(f"    outputs bitwise equal: {same}", flush=True)
    assert all(same)


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_workspace_not_16_byte_aligned(gpu_lib, kind):
    """A workspace 4 bytes past a 16-byte boundary: the partial rows are
    stored one element at a time instead of in 16-byte stores (same values)."""
    run_case(gpu_lib, kind, 700, 4096, "bf16", "bf16", seed=431, ws_offset=1)
    run_case(gpu_lib, kind, 700, 1024, "f32", "f32", seed=432, ws_offset=1)


def test_batch1_and_batch7(gpu_lib):
    for kind in ("ln", "rms"):
        run_case(gpu_lib, kind, 1, 4096, "bf16", "bf16", seed=430)
        run_case(gpu_lib, kind, 7, 4096, "bf16", "bf16", seed=430)


def test_large_offset_rows(gpu_lib):
    """Rows far from zero (x = 1000 + N(0, 1) in fp32): the two-pass variance keeps
    LayerNorm accurate where E[x^2] - mu^2 would cancel catastrophically."""
    run_case(gpu_lib, "ln", 9, 2048, "f32", "f32", seed=431, shift=1000.0)
    run_case(gpu_lib, "ln", 9, 2048, "f32", "f32", seed=431, shift=1000.0, saved=False)


def test_constant_rows_eps(gpu_lib):
    """A constant row has variance 0: rstd = 1 / sqrt(eps), y = b, finite gradients."""
    rows, cols = 3, 256
    x = np.full((rows, cols), 2.5, np.float32)
    w = np.ones(cols, np.float32)
    b = np.linspace(-1, 1, cols).astype(np.float32)
    y, mu, rstd = gpu_lib.vjp_layernorm_fwd(padded(x, "f32"), to_dev(w, "f32"), to_dev(b, "f32"), 1e-5)
    torch.cuda.synchronize()
    assert torch.allclose(y.cpu(), torch.from_numpy(np.tile(b, (rows, 1))), atol=1e-6)
    assert torch.allclose(rstd.cpu(), torch.full((rows,), 1e-5 ** -0.5), rtol=1e-6)


def test_empty(gpu_lib):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    y, mu, rstd = gpu_lib.vjp_layernorm_fwd(x, w, w)
    dw = torch.full((64,), 3.0, device=DEV)
    db = torch.full((64,), 4.0, device=DEV)
    gpu_lib.vjp_layernorm_bwd(x, x, w, mu, rstd, dw=dw, db=db, accumulate=True)
    gpu_lib.vjp_rmsnorm_bwd(x, x, w, None, dw=dw, accumulate=False)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and bool((db == 4.0).all()) and bool((dw == 0.0).all())


def test_too_wide_is_rejected(gpu_lib):
    x = torch.zeros((2, 16385), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(16385, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(gpu_lib.VjpError):
        gpu_lib.vjp_rmsnorm_fwd(x, w)


def test_deterministic(gpu_lib):
    x, w, b, dy = _inputs(3000, 1024, "bf16", "bf16", 440)
    xd, dyd, wd = to_dev(x, "bf16").view(3000, 1024), to_dev(dy, "bf16").view(3000, 1024), to_dev(w, "bf16")
    outs = [gpu_lib.vjp_rmsnorm_bwd(dyd, xd, wd) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][0], outs[1][0])


@pytest.mark.parametrize("kind", ["ln", "rms"])
def test_full_size(gpu_lib, kind):
    """32768 x 4096 bf16 (the softmax workload's shape): y and dx on every row
    against the oracle (in chunks of 1024 rows), dw (and db) over all rows."""
    rows, cols = 32768, 4096
    rms = kind == "rms"
    eps = 1e-6 if rms else 1e-5
    print(f"\n[{kind} full] {rows}x{cols}", flush=True)
    x, w, b, dy = _inputs(rows, cols, "bf16", "bf16", 450)
    xd, dyd = to_dev(x, "bf16").view(rows, cols), to_dev(dy, "bf16").view(rows, cols)
    wd, bd = to_dev(w, "bf16"), to_dev(b, "bf16")
    if rms:
        y, rstd = gpu_lib.vjp_rmsnorm_fwd(xd, wd, eps)
        dx, dw = gpu_lib.vjp_rmsnorm_bwd(dyd, xd, wd, rstd, eps)
    else:
        y, mu, rstd = gpu_lib.vjp_layernorm_fwd(xd, wd, bd, eps)
        dx, dw, db = gpu_lib.vjp_layernorm_bwd(dyd, xd, wd, mu, rstd, eps)
    torch.cuda.synchronize()
    y_host, dx_host = to_host(y, "bf16"), to_host(dx, "bf16")
    del y, dx, xd, dyd
    w64, b64 = synth.to_f64(w, "bf16"), synth.to_f64(b, "bf16")

    def part(i, j):
        xc, dyc = synth.to_f64(x[i:j], "bf16"), synth.to_f64(dy[i:j], "bf16")
        y_ref = nm.rmsnorm_fwd(xc, w64, eps)[0] if rms else nm.layernorm_fwd(xc, w64, b64, eps)[0]
        r_y = _check(y_host[i:j], y_ref, fwd_bound(xc, w64, b64, eps, rms), "bf16", "y")
        # the GPU's own fp32 statistics fed the backward: bound them as recomputed
        if rms:
            dx_ref, a1 = nm.rmsnorm_bwd(dyc, xc, w64, eps)[:2]
            a2 = np.zeros(cols)
            xhat = xc * nm.rmsnorm_rstd(xc, eps)[:, None]
        else:
            dx_ref, a1, a2 = nm.layernorm_bwd(dyc, xc, w64, eps)
            mu, rs = nm.layernorm_stats(xc, eps)
            xhat = (xc - mu[:, None]) * rs[:, None]
        r_dx = _check(dx_host[i:j], dx_ref, bwd_bound(dyc, xc, w64, eps, rms, saved=False), "bf16", "dx")
        return r_y, r_dx, a1, a2, np.sum(np.abs(dyc * xhat), axis=0), np.sum(np.abs(dyc), axis=0)

    parts = chunked(part, rows, 1024)
    reps = [combine([p[0] for p in parts], "y(all rows)"), combine([p[1] for p in parts], "dx(all rows)")]
    dw_ref, db_ref = sum(p[2] for p in parts), sum(p[3] for p in parts)
    S_dw, S_db = sum(p[4] for p in parts), sum(p[5] for p in parts)     # sums of |terms|
    reps.append(reduced(to_host(dw, "f32"), dw_ref, name="dw", S=S_dw))
    if not rms:
        reps.append(reduced(to_host(db, "f32"), db_ref, name="db", S=S_db))
    for r in reps:
        print("   ", r, flush=True)
    assert reps[0].n == rows * cols and reps[1].n == rows * cols
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]
