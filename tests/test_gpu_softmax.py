"""Row softmax forward / backward on the GPU vs the CPU oracle (calls the C ABI).

The backward is checked on a y produced by the oracle (forward rounded once to
the dtype), never on the GPU's own y.

dx tolerance: fp32 outputs use 1e-5 * max(|o|, S) with
S = |y| (|dy| + |s| + sum_k |dy_k y_k|), the magnitudes entering
y (dy - s) with s itself a sum; 16-bit outputs use 2 ulp, or where dy - s
cancels 2 ulp(o) + |y| (8 u (|dy| + |s|) + 1e-5 sum_k |dy_k y_k|).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, chunked, empty_padded, padded, to_host
from oracle.compare import U32, combine, pointwise
from oracle.rounding import round_to, to_storage
from synth.workloads import SOFTMAX

pytestmark = pytest.mark.gpu
sm = oracle.softmax


def _dx_tols(dy64, y64):
    s = np.sum(dy64 * y64, axis=-1, keepdims=True)
    sabs = np.sum(np.abs(dy64 * y64), axis=-1, keepdims=True)
    S = np.abs(y64) * (np.abs(dy64) + np.abs(s) + sabs)
    F = np.abs(y64) * (8 * U32 * (np.abs(dy64) + np.abs(s)) + 1e-5 * sabs)
    return S, F


def run_case(rwb, rows, cols, act, seed, sigma=3.0, ld=None, offset=0):
    print(f"\n[softmax] rows={rows} cols={cols} act={act} ld={ld} off={offset}", flush=True)
    x = synth.normal((rows, cols), sigma, act, seed, synth.STREAM_X)
    dy = synth.normal((rows, cols), 1.0, act, seed, synth.STREAM_DY)
    x64, dy64 = synth.to_f64(x, act), synth.to_f64(dy, act)
    xd = padded(x, act, ld, offset)
    y, ybuf = empty_padded(rows, cols, act, ld, offset)
    rwb.vjp_softmax_fwd(xd, y=y)
    y_ref = sm.fwd(x64)
    rep_y = pointwise(to_host(y, act), y_ref, act, name="y")
    # backward from the oracle's saved y (rounded once to the dtype)
    y_saved = to_storage(round_to(y_ref, act), act)
    y_saved64 = synth.to_f64(y_saved, act)
    yd = padded(y_saved, act, ld, offset)
    dyd = padded(dy, act, ld, offset)
    dx, dxbuf = empty_padded(rows, cols, act, ld, offset)
    rwb.vjp_softmax_bwd(dyd, yd, dx=dx)
    S, F = _dx_tols(dy64, y_saved64)
    rep_dx = pointwise(to_host(dx, act), sm.bwd(dy64, y_saved64), act, S=S, floor=F, name="dx")
    # nothing written before, after or between the rows of either output
    assert ybuf.intact() and dxbuf.intact(), "write outside an output"
    for r in (rep_y, rep_dx):
        print("   ", r, flush=True)
    assert rep_y.ok and rep_dx.ok, [str(rep_y), str(rep_dx)]


# cols chosen around the resident capacities (512 / 1024 / 2048 / 4096 per wave
# for 16-byte vectors) and beyond the resident limit (streaming path)
COLS16 = [1, 7, 100, 511, 512, 513, 4095, 4096, 4097, 8192, 20000, 32768, 40000]
COLS32 = [1, 7, 100, 2048, 2049, 16384, 17000]


@pytest.mark.parametrize("cols", COLS16)
@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_cols_16bit(gpu_lib, cols, act):
    rows = 7 if cols > 4096 else 33
    run_case(gpu_lib, rows, cols, act, seed=50 + cols)


@pytest.mark.parametrize("cols", COLS32)
def test_cols_f32(gpu_lib, cols):
    run_case(gpu_lib, 7, cols, "f32", seed=60 + cols)


@pytest.mark.parametrize("cols", [7, 4096, 4095, 40000])
@pytest.mark.parametrize("layout", ["padded_ld", "unaligned"])
def test_layouts(gpu_lib, cols, layout):
    ld, off = (cols + 8, 0) if layout == "padded_ld" else (cols + 1, 1)
    run_case(gpu_lib, 5, cols, "bf16", seed=70 + cols, ld=ld, offset=off)


def test_batch1_and_batch7(gpu_lib):
    run_case(gpu_lib, 1, 4096, "bf16", seed=80)
    run_case(gpu_lib, 7, 4096, "bf16", seed=80)


def test_shift_and_extremes(gpu_lib):
    """Large common shifts (shift invariance), a dominant logit, and a spread wide
    enough to make subnormal outputs (the no-flush exponential path)."""
    rows, cols = 6, 1000
    g = np.random.default_rng(3)
    x = (g.standard_normal((rows, cols)) * 3).astype(np.float32)
    x[0] += 1000.0
    x[1] -= 3000.0
    x[2, 17] = 80.0
    x[3, :] = np.linspace(-200, 0, cols)
    x[4, :] = 0.0
    x[5, :] = np.linspace(-95, 0, cols)
    xs = synth.f32_to_storage(x, "f32")
    xd = padded(xs, "f32")
    y = gpu_lib.vjp_softmax_fwd(xd)
    rep = pointwise(to_host(y, "f32"), sm.fwd(synth.to_f64(xs, "f32")), "f32", name="y(f32)")
    xb = synth.f32_to_storage(x, "bf16")
    yb = gpu_lib.vjp_softmax_fwd(padded(xb, "bf16"))
    rep_b = pointwise(to_host(yb, "bf16"), sm.fwd(synth.to_f64(xb, "bf16")), "bf16", name="y(bf16)")
    print("   ", rep, "\n   ", rep_b, flush=True)
    assert rep.ok and rep_b.ok


def test_empty(gpu_lib):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    y = gpu_lib.vjp_softmax_fwd(x)
    dx = gpu_lib.vjp_softmax_bwd(x, y)
    torch.cuda.synchronize()
    assert y.shape == (0, 64) and dx.shape == (0, 64)


def test_full_size(gpu_lib):
    """The 32768 x 4096 bf16 workload: y on every row against the oracle; dx on
    every row from the oracle's bf16 y (compared in chunks of 4096 rows)."""
    c = SOFTMAX
    rows, cols = c.shape
    print(f"\n[softmax full] {rows}x{cols}", flush=True)
    x = synth.normal((rows, cols), c.sigma_x, c.dtype, c.seed, synth.STREAM_X)
    dy = synth.normal((rows, cols), c.sigma_dy, c.dtype, c.seed, synth.STREAM_DY)
    xd = padded(x, "bf16")
    y, yg = empty_padded(rows, cols, "bf16")
    gpu_lib.vjp_softmax_fwd(xd, y=y)
    y_host = to_host(y, "bf16")
    assert yg.intact(), "write outside y"
    del xd, y
    y_saved = np.empty_like(x)

    def fwd_part(i, j):
        y_ref = sm.fwd(synth.to_f64(x[i:j], "bf16"))
        y_saved[i:j] = to_storage(round_to(y_ref, "bf16"), "bf16")
        return pointwise(y_host[i:j], y_ref, "bf16", name="y")

    r_y = chunked(fwd_part, rows, 2048)
    del y_host
    dx, dxg = empty_padded(rows, cols, "bf16")
    gpu_lib.vjp_softmax_bwd(padded(dy, "bf16"), padded(y_saved, "bf16"), dx=dx)
    dx_host = to_host(dx, "bf16")
    assert dxg.intact(), "write outside dx"

    def bwd_part(i, j):
        ys64, dys64 = synth.to_f64(y_saved[i:j], "bf16"), synth.to_f64(dy[i:j], "bf16")
        S, F = _dx_tols(dys64, ys64)
        return pointwise(dx_host[i:j], sm.bwd(dys64, ys64), "bf16", S=S, floor=F, name="dx")

    r_dx = chunked(bwd_part, rows, 2048)
    rep_y, rep_dx = combine(r_y, "y(all rows)"), combine(r_dx, "dx(all rows)")
    print("   ", rep_y, "\n   ", rep_dx, flush=True)
    assert rep_y.n == rows * cols and rep_dx.n == rows * cols
    assert rep_y.ok and rep_dx.ok
