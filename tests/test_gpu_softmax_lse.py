"""Softmax with saved row logsumexp (forward writes L, backward rebuilds y from
x and L) on the GPU vs the CPU oracle, through the C ABI.

The backward's L is the oracle's, rounded to fp32, so no GPU output feeds a
checked GPU input (a chained GPU forward -> backward case is checked too).

Tolerances.  L: 1e-5 * max(|L|, |m| + |L - m|).  dx: as for the saved-y
backward (S = |y| (|dy| + |s| + sum_k |dy_k y_k|), 16-bit floor
F = |y| (8 u (|dy| + |s|) + 1e-5 sum_k |dy_k y_k|)) plus the error of
rebuilding y = 2^((x - L) log2 e) in fp32: relative delta = 4 u (2 + |a| + |L|)
with a = (x - L) log2 e (rounding of x - L, of the product, of the stored L
and of the exponential), entering dx through y and through s.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, Guarded, chunked, empty_padded, padded, pick_rows, to_host
from oracle.compare import U32, combine, pointwise
from synth.workloads import SOFTMAX

pytestmark = pytest.mark.gpu
sm = oracle.softmax


def _lse_S(x64):
    m = np.max(x64, axis=-1)
    L = sm.lse(x64)
    return np.abs(m) + np.abs(L - m)


def _dx_tols(dy64, x64, L32):
    y = sm.fwd(x64)
    s = np.sum(dy64 * y, axis=-1, keepdims=True)
    sabs = np.sum(np.abs(dy64 * y), axis=-1, keepdims=True)
    a = (x64 - L32[:, None]) * np.log2(np.e)
    delta = 4 * U32 * (2 + np.abs(a) + np.abs(L32)[:, None])
    dmax = np.max(delta, axis=-1, keepdims=True)
    S0 = np.abs(y) * (np.abs(dy64) + np.abs(s) + sabs)
    S = S0 * np.maximum(1.0, (delta + dmax + 8 * U32) / 1e-5)
    F = np.abs(y) * (8 * U32 * (np.abs(dy64) + np.abs(s)) + 1e-5 * sabs) \
        + np.abs(y) * (delta * (np.abs(dy64) + np.abs(s)) + dmax * sabs)
    return S, F


def run_case(rwb, rows, cols, act, seed, sigma=3.0, ld=None, offset=0):
    print(f"\n[softmax_lse] rows={rows} cols={cols} act={act} ld={ld} off={offset}", flush=True)
    x = synth.normal((rows, cols), sigma, act, seed, synth.STREAM_X)
    dy = synth.normal((rows, cols), 1.0, act, seed, synth.STREAM_DY)
    x64, dy64 = synth.to_f64(x, act), synth.to_f64(dy, act)
    xd = padded(x, act, ld, offset)
    y, _ = empty_padded(rows, cols, act, ld, offset)
    lse_g = Guarded(rows, torch.float32)
    rwb.vjp_softmax_fwd_lse(xd, y=y, row_lse=lse_g.t)
    lse_only = Guarded(rows, torch.float32)
    rwb.vjp_softmax_fwd_lse(xd, row_lse=lse_only.t, write_y=False)
    torch.cuda.synchronize()
    assert lse_g.intact() and lse_only.intact()
    L_ref = sm.lse(x64)
    reps = [pointwise(to_host(y, act), sm.fwd(x64), act, name="y"),
            pointwise(to_host(lse_g.t, "f32"), L_ref, "f32", S=_lse_S(x64), name="row_lse")]
    assert torch.equal(lse_g.t, lse_only.t), "statistics-only forward differs"
    # backward from the oracle's L (fp32)
    L32 = L_ref.astype(np.float32)
    dyd = padded(dy, act, ld, offset)
    dx, _ = empty_padded(rows, cols, act, ld, offset)
    rwb.vjp_softmax_bwd_lse(dyd, xd, torch.from_numpy(L32).to(DEV), dx=dx)
    S, F = _dx_tols(dy64, x64, L32.astype(np.float64))
    reps.append(pointwise(to_host(dx, act), sm.bwd_from_x(dy64, x64), act, S=S, floor=F, name="dx"))
    # chained: the GPU's own L feeds the GPU backward
    dx2, _ = empty_padded(rows, cols, act, ld, offset)
    rwb.vjp_softmax_bwd_lse(dyd, xd, lse_g.t, dx=dx2)
    S2, F2 = _dx_tols(dy64, x64, to_host(lse_g.t, "f32").astype(np.float64))
    reps.append(pointwise(to_host(dx2, act), sm.bwd_from_x(dy64, x64), act, S=S2, floor=F2,
                          name="dx(chained)"))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


COLS16 = [1, 7, 100, 512, 513, 4095, 4096, 4097, 8192, 20000, 32768, 40000]


@pytest.mark.parametrize("cols", COLS16)
@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_cols_16bit(gpu_lib, cols, act):
    run_case(gpu_lib, 7 if cols > 4096 else 33, cols, act, seed=150 + cols)


@pytest.mark.parametrize("cols", [1, 7, 2048, 2049, 16384, 17000])
def test_cols_f32(gpu_lib, cols):
    run_case(gpu_lib, 7, cols, "f32", seed=160 + cols)


@pytest.mark.parametrize("cols", [7, 4095, 40000])
@pytest.mark.parametrize("layout", ["padded_ld", "unaligned"])
def test_layouts(gpu_lib, cols, layout):
    ld, off = (cols + 8, 0) if layout == "padded_ld" else (cols + 1, 1)
    run_case(gpu_lib, 5, cols, "bf16", seed=170 + cols, ld=ld, offset=off)


def test_batch1_and_batch7(gpu_lib):
    run_case(gpu_lib, 1, 4096, "bf16", seed=180)
    run_case(gpu_lib, 7, 4096, "bf16", seed=180)


def test_extremes(gpu_lib):
    """Large shifts, a dominant logit, and spreads that make subnormal probabilities."""
    rows, cols = 6, 1000
    g = np.random.default_rng(4)
    x = (g.standard_normal((rows, cols)) * 3).astype(np.float32)
    x[0] += 1000.0
    x[1] -= 3000.0
    x[2, 17] = 80.0
    x[3, :] = np.linspace(-200, 0, cols)
    x[4, :] = 0.0
    x[5, :] = np.linspace(-95, 0, cols)
    dy = g.standard_normal((rows, cols)).astype(np.float32)
    for act in ("f32", "bf16"):
        xs, dys = synth.f32_to_storage(x, act), synth.f32_to_storage(dy, act)
        x64, dy64 = synth.to_f64(xs, act), synth.to_f64(dys, act)
        xd = padded(xs, act)
        _, L = gpu_lib.vjp_softmax_fwd_lse(xd, write_y=False)
        rep_l = pointwise(to_host(L, "f32"), sm.lse(x64), "f32", S=_lse_S(x64), name=f"lse({act})")
        L32 = sm.lse(x64).astype(np.float32)
        dx = gpu_lib.vjp_softmax_bwd_lse(padded(dys, act), xd, torch.from_numpy(L32).to(DEV))
        S, F = _dx_tols(dy64, x64, L32.astype(np.float64))
        rep_d = pointwise(to_host(dx, act), sm.bwd_from_x(dy64, x64), act, S=S, floor=F,
                          name=f"dx({act})")
        print("   ", rep_l, "\n   ", rep_d, flush=True)
        assert rep_l.ok and rep_d.ok


def test_empty(gpu_lib):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    y, L = gpu_lib.vjp_softmax_fwd_lse(x)
    dx = gpu_lib.vjp_softmax_bwd_lse(x, x, L)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and L.shape == (0,) and dx.shape == (0, 64)


def test_full_size(gpu_lib):
    """The 32768 x 4096 bf16 workload: y and L on every row, then the backward
    from the oracle's L on every row (compared in chunks of 2048 rows)."""
    c = SOFTMAX
    rows, cols = c.shape
    print(f"\n[softmax_lse full] {rows}x{cols}", flush=True)
    x = synth.normal((rows, cols), c.sigma_x, c.dtype, c.seed, synth.STREAM_X)
    dy = synth.normal((rows, cols), c.sigma_dy, c.dtype, c.seed, synth.STREAM_DY)
    xd = padded(x, "bf16")
    y, L = gpu_lib.vjp_softmax_fwd_lse(xd)
    y_host, L_host = to_host(y, "bf16"), to_host(L, "f32")
    del y
    L_ref = np.empty(rows)

    def fwd_part(i, j):
        xs = synth.to_f64(x[i:j], "bf16")
        L_ref[i:j] = sm.lse(xs)
        return (pointwise(y_host[i:j], sm.fwd(xs), "bf16", name="y"),
                pointwise(L_host[i:j], L_ref[i:j], "f32", S=_lse_S(xs), name="lse"))

    r_fwd = chunked(fwd_part, rows, 2048)
    del y_host
    L32 = L_ref.astype(np.float32)
    dx = gpu_lib.vjp_softmax_bwd_lse(padded(dy, "bf16"), xd, torch.from_numpy(L32).to(DEV))
    dx_host = to_host(dx, "bf16")
    del dx

    def bwd_part(i, j):
        xs, dys = synth.to_f64(x[i:j], "bf16"), synth.to_f64(dy[i:j], "bf16")
        S, F = _dx_tols(dys, xs, L32[i:j].astype(np.float64))
        return pointwise(dx_host[i:j], sm.bwd_from_x(dys, xs), "bf16", S=S, floor=F, name="dx")

    r_dx = chunked(bwd_part, rows, 2048)
    reps = [combine([r[0] for r in r_fwd], "y(all rows)"), combine([r[1] for r in r_fwd], "lse(all rows)"),
            combine(r_dx, "dx(all rows)")]
    for r in reps:
        print("   ", r, flush=True)
    assert reps[0].n == rows * cols and reps[1].n == rows and reps[2].n == rows * cols
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]
