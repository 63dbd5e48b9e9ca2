"""Weighted sum on the GPU vs the CPU oracle, element by element (calls the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, Guarded, chunked, empty_padded, padded, to_dev, to_host
from oracle.compare import U32, combine, exact, pointwise, reduced
from synth.workloads import WS_LARGE, WS_SMALL

pytestmark = pytest.mark.gpu
ws = oracle.weighted_sum


def _inputs(n, d, act, wdt, seed, sigma_w=1.0):
    x = synth.normal((n, d), 1.0, act, seed, synth.STREAM_X)
    w = synth.normal((d,), sigma_w, wdt, seed, synth.STREAM_W)
    dy = synth.normal((n,), 1.0, act, seed, synth.STREAM_DY)
    return x, w, dy


def _dx_is_one_rounding(act, wdt):
    # dy * w is exact in fp32 unless a 16-bit activation meets an fp32 weight
    return act == "f32" or wdt != "f32"


def run_case(rwb, n, d, act, wdt, seed, ld=None, offset=0, rows_per_tile=0, accumulate=False,
             w_offset=0):
    x, w, dy = _inputs(n, d, act, wdt, seed)
    x64, w64, dy64 = synth.to_f64(x, act), synth.to_f64(w, wdt), synth.to_f64(dy, act)
    print(f"\n[weighted_sum] n={n} d={d} act={act} w={wdt} ld={ld} off={offset} "
          f"rpt={rows_per_tile} acc={accumulate}", flush=True)
    xd = padded(x, act, ld, offset)
    if w_offset:   # w starting w_offset elements into its buffer (not 16-byte aligned)
        wbuf = torch.zeros(d + w_offset, dtype=synth.torch_dtype(wdt), device=DEV)
        wbuf[w_offset:] = to_dev(w, wdt)
        wd = wbuf[w_offset:]
    else:
        wd = to_dev(w, wdt)
    dyd = to_dev(dy, act)
    yg = Guarded(n, synth.torch_dtype(act))
    rwb.vjp_weighted_sum_fwd(xd, wd, y=yg.t)
    dx, _ = empty_padded(n, d, act, ld, offset)
    g = np.random.default_rng(seed)
    old = g.standard_normal(d).astype(np.float32)
    dwg = Guarded(d, torch.float32, fill=0.0)
    if accumulate:
        dwg.t.copy_(torch.from_numpy(old))
    need = rwb.vjp_weighted_sum_bwd_workspace_size(n, d, rows_per_tile)
    wsg = Guarded(need // 4, torch.float32)
    rwb.vjp_weighted_sum_bwd(dyd, xd, wd, dx=dx, dw=dwg.t, accumulate=accumulate,
                             rows_per_tile=rows_per_tile, workspace=wsg.t)
    torch.cuda.synchronize()
    assert yg.intact() and dwg.intact() and wsg.intact(), "write outside an output"

    reps = []
    S = ws.fwd(np.abs(x64), np.abs(w64))
    reps.append(pointwise(to_host(yg.t, act), ws.fwd(x64, w64), act, S=S,
                          floor=d * U32 * S, name="y"))
    gx_ref, gw_ref = ws.bwd(dy64, x64, w64, grad_w_old=old.astype(np.float64) if accumulate else None)
    from oracle.rounding import round_to, to_storage
    dx_host = to_host(dx, act)
    if _dx_is_one_rounding(act, wdt):
        reps.append(exact(dx_host, to_storage(round_to(gx_ref, act), act), act, name="dx"))
    else:
        reps.append(pointwise(dx_host, gx_ref, act, name="dx"))
    reps.append(reduced(to_host(dwg.t, "f32"), gw_ref, name="dw"))
    br, tiles = rwb.vjp_weighted_sum_tiling(n, rows_per_tile)
    if n > 0 and d > 0:
        P = to_host(wsg.t, "f32").reshape(-1, d)
        P_ref = ws.partials(x64, dy64, br, tiles)
        assert P.shape == P_ref.shape
        reps.append(pointwise(P, P_ref, "f32", S=ws.partials(np.abs(x64), np.abs(dy64), br, tiles),
                              name="partials"))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]
    return reps


def test_worked_tiling_case(gpu_lib):
    """100 rows, tiles of 32 rows, D = 64, fp32: four partial rows of 64, then grad_w [64]."""
    c = WS_SMALL
    assert gpu_lib.vjp_weighted_sum_bwd_workspace_size(100, 64, 32) == 4 * 64 * 4
    run_case(gpu_lib, 100, 64, "f32", "f32", c.seed, rows_per_tile=32)
    run_case(gpu_lib, 100, 64, "f32", "f32", c.seed, rows_per_tile=32, accumulate=True)


SHAPES = [(1, 1), (7, 7), (7, 64), (1, 256), (333, 256), (1000, 100), (257, 600), (64, 1030),
          (2049, 33), (9, 8193), (3, 50001)]
DTYPES = [("f32", "f32"), ("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"), ("f16", "f32"),
          ("f32", "bf16")]


@pytest.mark.parametrize("n,d", SHAPES)
@pytest.mark.parametrize("act,wdt", DTYPES)
def test_shapes_dtypes(gpu_lib, n, d, act, wdt):
    run_case(gpu_lib, n, d, act, wdt, seed=7 + n + d)


@pytest.mark.parametrize("n,d", [(7, 64), (333, 256), (257, 600)])
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("layout", ["padded_ld", "unaligned"])
def test_layouts(gpu_lib, n, d, act, layout):
    ld, off = (d + 8, 0) if layout == "padded_ld" else (d + 1, 1)
    run_case(gpu_lib, n, d, act, act, seed=11 + d, ld=ld, offset=off)


@pytest.mark.parametrize("rpt", [1, 7, 32, 100, 5000])
def test_rows_per_tile(gpu_lib, rpt):
    run_case(gpu_lib, 1000, 64, "bf16", "bf16", seed=13, rows_per_tile=rpt, accumulate=True)


@pytest.mark.parametrize("n,d", [(32768 + 32 * 9 + 5, 64), (70001, 256), (131072, 40)])
def test_round_robin_tiles(gpu_lib, n, d):
    """Automatic tiling past 1024 blocks: several blocks per tile, a ragged last block."""
    br, tiles = gpu_lib.vjp_weighted_sum_tiling(n, 0)
    assert br == 32 and tiles == 1024
    run_case(gpu_lib, n, d, "bf16", "bf16", seed=19 + n, accumulate=True)


def test_batch1_vs_batch7(gpu_lib):
    """A missing batch reduction passes at batch 1 and fails at batch 7."""
    run_case(gpu_lib, 1, 64, "f32", "f32", seed=17)
    run_case(gpu_lib, 7, 64, "f32", "f32", seed=17)


def test_empty_batch(gpu_lib):
    x = torch.empty((0, 64), dtype=torch.float32, device=DEV)
    w = torch.ones(64, dtype=torch.float32, device=DEV)
    y = gpu_lib.vjp_weighted_sum_fwd(x, w)
    assert y.shape == (0,)
    dw = torch.full((64,), 3.0, device=DEV)
    gpu_lib.vjp_weighted_sum_bwd(torch.empty(0, device=DEV), x, w, dw=dw, accumulate=True)
    torch.cuda.synchronize()
    assert bool((dw == 3.0).all())
    gpu_lib.vjp_weighted_sum_bwd(torch.empty(0, device=DEV), x, w, dw=dw, accumulate=False)
    torch.cuda.synchronize()
    assert bool((dw == 0.0).all())


def test_zero_width_rows(gpu_lib):
    """d = 0: every y is an empty sum (0), grad_x and grad_w are empty."""
    x = torch.empty((5, 0), dtype=torch.bfloat16, device=DEV)
    w = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    y = torch.full((5,), 7.0, dtype=torch.bfloat16, device=DEV)
    gpu_lib.vjp_weighted_sum_fwd(x, w, y=y)
    dx, dw = gpu_lib.vjp_weighted_sum_bwd(torch.ones(5, dtype=torch.bfloat16, device=DEV), x, w)
    torch.cuda.synchronize()
    assert bool((y == 0).all()) and dx.shape == (5, 0) and dw.shape == (0,)


def test_large_batch_full_size(gpu_lib):
    """The 1,048,576 x 256 bf16 workload in the benchmark's launch configuration:
    y and grad_x on every row (in chunks), grad_w and every tile partial in
    full; grad_w's condition number is reported."""
    c = WS_LARGE
    n, d = c.shape
    x = synth.normal((n, d), c.sigma_x, c.dtype, c.seed, synth.STREAM_X)
    w = synth.normal((d,), c.sigma_w, c.w_dtype, c.seed, synth.STREAM_W)
    dy = synth.normal((n,), c.sigma_dy, c.dtype, c.seed, synth.STREAM_DY)
    print(f"\n[weighted_sum full] {n}x{d} bf16", flush=True)
    xd, wd, dyd = to_dev(x, "bf16").view(n, d), to_dev(w, "bf16"), to_dev(dy, "bf16")
    yg = Guarded(n, torch.bfloat16)
    gpu_lib.vjp_weighted_sum_fwd(xd, wd, y=yg.t)
    dx, dxg = empty_padded(n, d, "bf16")
    dwg = Guarded(d, torch.float32)
    br, tiles = gpu_lib.vjp_weighted_sum_tiling(n, 0)
    need = gpu_lib.vjp_weighted_sum_bwd_workspace_size(n, d, 0)
    wsg = Guarded(need // 4, torch.float32)
    gpu_lib.vjp_weighted_sum_bwd(dyd, xd, wd, dx=dx, dw=dwg.t, workspace=wsg.t)
    dx2, dw2 = gpu_lib.vjp_weighted_sum_bwd(dyd, xd, wd)
    torch.cuda.synchronize()
    assert (br, tiles) == (32, 1024) and need == 1024 * 256 * 4
    assert yg.intact() and dxg.intact() and dwg.intact() and wsg.intact(), "write outside an output"
    # determinism: a second call (its own workspace), bitwise identical
    assert torch.equal(dwg.t, dw2) and torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    del dx2

    from oracle.rounding import round_to, to_storage
    w64, dy64 = synth.to_f64(w, "bf16"), synth.to_f64(dy, "bf16")
    y_host, dx_host = to_host(yg.t, "bf16"), to_host(dx, "bf16")
    # grad_w and the stage-1 partials over all rows, from the oracle's partials:
    # a chunk of br * tiles rows starts at block 0 of the round-robin, so the
    # partials of the chunks add tile by tile
    chunk = br * tiles

    def part(i, j):
        xc = synth.to_f64(x[i:j], "bf16")
        S = ws.fwd(np.abs(xc), np.abs(w64))
        ry = pointwise(y_host[i:j], ws.fwd(xc, w64), "bf16", S=S, floor=d * U32 * S, name="y")
        gx_ref, _ = ws.bwd(dy64[i:j], xc, w64)
        rdx = exact(dx_host[i:j], to_storage(round_to(gx_ref, "bf16"), "bf16"), "bf16", name="dx")
        return (ry, rdx, ws.partials(xc, dy64[i:j], br, tiles),
                ws.partials(np.abs(xc), np.abs(dy64[i:j]), br, tiles))

    parts = chunked(part, n, chunk)
    r_y, r_dx = [q[0] for q in parts], [q[1] for q in parts]
    P_ref = np.sum([q[2] for q in parts], axis=0)
    Pa = np.sum([q[3] for q in parts], axis=0)
    reps = [combine(r_y, "y(all rows)"), combine(r_dx, "dx(all rows)")]
    reps.append(pointwise(to_host(wsg.t, "f32").reshape(-1, d), P_ref, "f32", S=Pa, name="partials"))
    reps.append(reduced(to_host(dwg.t, "f32"), P_ref.sum(axis=0), name="dw", S=Pa.sum(axis=0)))
    for r in reps:
        print("   ", r, flush=True)
    assert reps[0].n == n and reps[1].n == n * d
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


@pytest.mark.parametrize("wdt", ["bf16", "f16", "f32"])
def test_parameter_vector_alignment(gpu_lib, wdt):
    """16-byte aligned rows with w aligned (16-byte parameter loads) and w one
    element past a 16-byte boundary (one load per element): same results."""
    run_case(gpu_lib, 3000, 512, "bf16", wdt, seed=91)
    run_case(gpu_lib, 3000, 512, "bf16", wdt, seed=91, w_offset=1)
    run_case(gpu_lib, 700, 300, "f32", wdt, seed=92, w_offset=1)


@pytest.mark.parametrize("act, wdt", [("bf16", "bf16"), ("bf16", "f16"), ("bf16", "f32"),
                                      ("f32", "bf16"), ("f32", "f32")])
def test_parameter_loads_same_bits(gpu_lib, act, wdt):
    """w at a 16-byte boundary (vector loads) and one element past it
    (element loads): y, grad_x and grad_w bit for bit the same."""
    n, d = 3000, 512
    print(f"\n[weighted_sum parameter loads] n={n} d={d} act={act} w={wdt}", flush=True)
    x, w, dy = _inputs(n, d, act, wdt, 93)
    xd, dyd = padded(x, act), to_dev(dy, act)
    outs = []
    for off in (0, 1):
        wbuf = torch.zeros(d + off, dtype=synth.torch_dtype(wdt), device=DEV)
        wbuf[off:] = to_dev(w, wdt)
        y = gpu_lib.vjp_weighted_sum_fwd(xd, wbuf[off:])
        dx, dw = gpu_lib.vjp_weighted_sum_bwd(dyd, xd, wbuf[off:])
        torch.cuda.synchronize()
        outs.append([t.cpu().view(torch.int16 if t.element_size() == 2 else torch.int32)
                     for t in (y, dx, dw)])
    same = [torch.equal(a, b) for a, b in zip(*outs)]
    print(f"    y, grad_x, grad_w bitwise equal: {same}", flush=True)
    assert all(same)


def test_widest_rows_unaligned(gpu_lib):
    """d = 4194240, the widest the backward takes: 65535 column blocks of 64
    in its one-element-per-load form (rows 2 bytes past a 16-byte boundary)."""
    run_case(gpu_lib, 3, 65535 * 64, "bf16", "bf16", 977, offset=1)
