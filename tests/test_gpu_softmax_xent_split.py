"""Split softmax-cross-entropy (statistics-only forward, backward that rebuilds
p = exp(z - lse) with a device upstream gradient) on the GPU vs the CPU
oracle, through the C ABI.

The backward's lse is the oracle's, rounded to fp32.  Tolerances as for the
fused form (row_max bitwise; lse and row losses 1e-5 * max(|o|, |m| +
|lse - m| (+ |z_t|)); mean loss 1e-4; n_invalid exact), and for dlogits the
fused rule plus the error of rebuilding p in fp32: relative
delta = 4 u (2 + |a| + |lse|), a = (z - lse) log2 e.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, Guarded, chunked, empty_padded, padded, pick_rows, to_host
from oracle.compare import U32, combine, exact, pointwise, reduced
from synth.workloads import XENT

pytestmark = pytest.mark.gpu
xe = oracle.softmax_xent


def _check_fwd(out, ws_rows, z64, t, has_max=True):
    ref = xe.fwd(z64, t)
    m, lse = ref["row_max"], ref["row_lse"]
    C = z64.shape[1]
    valid = (t >= 0) & (t < C)
    zt = np.where(valid, z64[np.arange(len(t)), np.clip(t, 0, C - 1)], 0)
    S_lse = np.abs(m) + np.abs(lse - m)
    reps = [pointwise(out["row_lse"], lse, "f32", S=S_lse, name="row_lse"),
            pointwise(ws_rows, ref["row_loss"], "f32", S=S_lse + np.abs(zt), name="row_loss"),
            reduced(out["loss"], np.array([ref["loss"]]), name="loss")]
    if has_max:
        reps.append(exact(out["row_max"], m.astype(np.float32), "f32", name="row_max"))
    return ref, reps


def _dz_tols_at(z_cols, cols, t, lse64, L32, scale):
    """Scale S and floor F of dlogits at columns `cols` (z_cols = z[:, cols])
    given the exact row lse and the fp32 lse the kernel was handed."""
    p = np.exp(z_cols - lse64[:, None])
    onehot = (np.asarray(cols)[None, :] == np.asarray(t)[:, None]).astype(np.float64)
    a = (z_cols - L32[:, None]) * np.log2(np.e)
    delta = 4 * U32 * (2 + np.abs(a) + np.abs(L32)[:, None])
    S = np.abs(scale) * (p + onehot) * np.maximum(1.0, (delta + 8 * U32) / 1e-5)
    F = 16 * U32 * np.abs(scale) * onehot + np.abs(scale) * p * delta
    return S, F


def _dz_tols(z64, t, L32, dloss, act):
    R, C = z64.shape
    return _dz_tols_at(z64, np.arange(C), t, xe.fwd(z64, t)["row_lse"], L32, dloss / R)


def run_case(rwb, rows, C, act, seed, sigma=2.0, ld=None, offset=0, targets=None, dloss=1.0,
             in_place=False, z=None):
    print(f"\n[xent split] rows={rows} C={C} act={act} ld={ld} off={offset} dloss={dloss} "
          f"in_place={in_place}", flush=True)
    if z is None:
        z = synth.normal((rows, C), sigma, act, seed, synth.STREAM_X)
    t = synth.targets(rows, C, seed) if targets is None else np.asarray(targets, np.int32)
    z64 = synth.to_f64(z, act)
    zd = padded(z, act, ld, offset)
    td = torch.from_numpy(t).to(DEV)
    loss, rmax, rlse = Guarded(1, torch.float32), Guarded(rows, torch.float32), Guarded(rows, torch.float32)
    ninv = Guarded(1, torch.int32)
    wsg = Guarded(rwb.vjp_softmax_xent_workspace_size(rows) // 4, torch.float32)
    rwb.vjp_softmax_xent_fwd(zd, td, loss=loss.t, row_lse=rlse.t, row_max=rmax.t, n_invalid=ninv.t,
                             workspace=wsg.t)
    torch.cuda.synchronize()
    assert loss.intact() and rmax.intact() and rlse.intact() and ninv.intact() and wsg.intact()
    out = {"row_lse": to_host(rlse.t, "f32"), "row_max": to_host(rmax.t, "f32"),
           "loss": to_host(loss.t, "f32")}
    ref, reps = _check_fwd(out, to_host(wsg.t, "f32"), z64, t)
    assert int(ninv.t.item()) == ref["n_invalid"]
    # backward from the oracle's lse and a device upstream gradient
    L32 = ref["row_lse"].astype(np.float32)
    dl = torch.tensor([dloss], dtype=torch.float32, device=DEV)
    if in_place:
        dz = zd
    else:
        dz, _ = empty_padded(rows, C, act, ld, offset)
    rwb.vjp_softmax_xent_bwd(zd, td, torch.from_numpy(L32).to(DEV), dl, dlogits=dz)
    S, F = _dz_tols(z64, t, L32.astype(np.float64), dloss, act)
    reps.append(pointwise(to_host(dz, act), xe.bwd(z64, t, dloss), act, S=S, floor=F, name="dlogits"))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


def spread_rows(C, act, seed):
    """Rows whose logits span 100 to 200 natural-log units: the smallest
    probabilities, and the gradients scale * p, fall in the subnormal range
    of fp32 / bf16 (no flush to zero on any path), beside a normal row."""
    g = np.random.default_rng(seed)
    z = np.empty((5, C), np.float32)
    z[0] = np.linspace(-100.0, 0.0, C)
    z[1] = np.linspace(-140.0, 10.0, C)
    z[2] = np.linspace(-90.0, -80.0, C)
    z[2, C // 2] = 0.0
    z[3] = g.standard_normal(C) * 2
    z[4] = np.linspace(-200.0, 0.0, C)
    return synth.f32_to_storage(g.permutation(z, axis=1), act)


COLS16 = [1, 2, 7, 1000, 4095, 4096, 32000, 32768, 40000, 70000]


@pytest.mark.parametrize("C", COLS16)
@pytest.mark.parametrize("act", ["bf16", "f16"])
def test_classes_16bit(gpu_lib, C, act):
    run_case(gpu_lib, 7 if C > 4096 else 37, C, act, seed=190 + C)


@pytest.mark.parametrize("C", [1, 7, 2048, 16384, 17000])
def test_classes_f32(gpu_lib, C):
    run_case(gpu_lib, 7, C, "f32", seed=195 + C)


@pytest.mark.parametrize("C", [7, 32000, 40000])
@pytest.mark.parametrize("layout", ["padded_ld", "unaligned"])
def test_layouts(gpu_lib, C, layout):
    ld, off = (C + 8, 0) if layout == "padded_ld" else (C + 1, 1)
    run_case(gpu_lib, 5, C, "bf16", seed=197 + C, ld=ld, offset=off)


@pytest.mark.parametrize("dloss", [0.0, -2.5, 3.0e4])
def test_upstream_gradient(gpu_lib, dloss):
    run_case(gpu_lib, 7, 32000, "bf16", seed=199, dloss=dloss)


@pytest.mark.parametrize("C,ld", [(32000, None), (1000, 1003)])
def test_in_place(gpu_lib, C, ld):
    run_case(gpu_lib, 9, C, "bf16", seed=201, ld=ld, in_place=True)


def test_invalid_targets(gpu_lib):
    run_case(gpu_lib, 6, 300, "bf16", seed=203, targets=[3, -1, 300, 0, 299, 2 ** 31 - 1])


@pytest.mark.parametrize("act,C", [("bf16", 300), ("f32", 301)])
def test_invalid_target_in_last_vector_padding(gpu_lib, act, C):
    run_case(gpu_lib, 4, C, act, seed=204, ld=304, targets=[3, C, 0, 303])


def test_batch1_and_batch7(gpu_lib):
    run_case(gpu_lib, 1, 32000, "bf16", seed=205)
    run_case(gpu_lib, 7, 32000, "bf16", seed=205)


def test_no_row_max(gpu_lib):
    """row_max is optional in the split forward."""
    z = synth.normal((5, 700), 2.0, "bf16", 207, synth.STREAM_X)
    t = synth.targets(5, 700, 207)
    out = gpu_lib.vjp_softmax_xent_fwd(padded(z, "bf16"), torch.from_numpy(t).to(DEV))
    torch.cuda.synchronize()
    assert out["row_max"] is None
    res = {"row_lse": to_host(out["row_lse"], "f32"), "loss": to_host(out["loss"], "f32")}
    ref = xe.fwd(synth.to_f64(z, "bf16"), t)
    S = np.abs(ref["row_max"]) + np.abs(ref["row_lse"] - ref["row_max"])
    r1 = pointwise(res["row_lse"], ref["row_lse"], "f32", S=S, name="row_lse")
    r2 = reduced(res["loss"], np.array([ref["loss"]]), name="loss")
    assert r1.ok and r2.ok


def test_matches_fused(gpu_lib):
    """With dloss = 1 the split backward and the fused form agree to rounding."""
    z = synth.normal((8, 32000), 2.0, "bf16", 209, synth.STREAM_X)
    t = synth.targets(8, 32000, 209)
    zd, td = padded(z, "bf16"), torch.from_numpy(t).to(DEV)
    fused = gpu_lib.vjp_softmax_xent_fwd_bwd(zd, td)
    split = gpu_lib.vjp_softmax_xent_fwd(zd, td, want_max=True)
    dz = gpu_lib.vjp_softmax_xent_bwd(zd, td, split["row_lse"], torch.ones(1, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(fused["row_lse"], split["row_lse"])
    assert torch.equal(fused["row_max"], split["row_max"])
    assert torch.equal(fused["loss"], split["loss"])
    a = fused["dlogits"].float()
    b = dz.float()
    assert float((a - b).abs().max()) <= float(2.0 ** -7 * a.abs().max())


def test_empty(gpu_lib):
    z = torch.empty((0, 10), dtype=torch.bfloat16, device=DEV)
    ti = torch.empty(0, dtype=torch.int32, device=DEV)
    out = gpu_lib.vjp_softmax_xent_fwd(z, ti)
    dz = gpu_lib.vjp_softmax_xent_bwd(z, ti, out["row_lse"], torch.ones(1, device=DEV))
    torch.cuda.synchronize()
    assert np.isnan(out["loss"].item()) and dz.shape == (0, 10)


def test_full_size(gpu_lib):
    """The 16384 x 32000 bf16 workload: the forward on every row (row_lse,
    row_max) and its mean loss, then dlogits on every row from the oracle's
    lse (compared in chunks of 512 rows)."""
    c = XENT
    rows, C = c.shape
    print(f"\n[xent split full] {rows}x{C}", flush=True)
    z = synth.normal((rows, C), c.sigma_x, c.dtype, c.seed, synth.STREAM_X)
    t = synth.targets(rows, C, c.seed)
    zd, td = padded(z, "bf16"), torch.from_numpy(t).to(DEV)
    wsb = torch.empty(gpu_lib.vjp_softmax_xent_workspace_size(rows) // 4, dtype=torch.float32, device=DEV)
    out = gpu_lib.vjp_softmax_xent_fwd(zd, td, want_max=True, workspace=wsb)
    lse_host, max_host = to_host(out["row_lse"], "f32"), to_host(out["row_max"], "f32")
    loss_host = to_host(out["loss"], "f32")
    L_ref, row_loss = np.empty(rows), np.empty(rows)

    def fwd_part(i, j):
        ref = xe.fwd(synth.to_f64(z[i:j], "bf16"), t[i:j])
        L_ref[i:j], row_loss[i:j] = ref["row_lse"], ref["row_loss"]
        S = np.abs(ref["row_max"]) + np.abs(ref["row_lse"] - ref["row_max"])
        return (pointwise(lse_host[i:j], ref["row_lse"], "f32", S=S, name="row_lse"),
                exact(max_host[i:j], ref["row_max"].astype(np.float32), "f32", name="row_max"))

    r_fwd = chunked(fwd_part, rows, 512)
    reps = [combine([r[0] for r in r_fwd], "row_lse(all rows)"),
            combine([r[1] for r in r_fwd], "row_max(all rows)"),
            reduced(loss_host, np.array([np.sum(row_loss) / rows]), name="loss",
                    S=[np.sum(np.abs(row_loss)) / rows])]
    L32 = L_ref.astype(np.float32)
    dz = gpu_lib.vjp_softmax_xent_bwd(zd, td, torch.from_numpy(L32).to(DEV), torch.ones(1, device=DEV))
    dz_host = to_host(dz, "bf16")
    del dz, zd

    def bwd_part(i, j):
        zs = synth.to_f64(z[i:j], "bf16")
        # _dz_tols and xe.bwd scale by dloss / (j - i): pass dloss so that the scale is 1 / rows
        dl = 1.0 * (j - i) / rows
        S, F = _dz_tols(zs, t[i:j], L32[i:j].astype(np.float64), dl, "bf16")
        return pointwise(dz_host[i:j], xe.bwd(zs, t[i:j], dl), "bf16", S=S, floor=F, name="dlogits")

    reps.append(combine(chunked(bwd_part, rows, 512), "dlogits(all rows)"))
    for r in reps:
        print("   ", r, flush=True)
    assert reps[0].n == rows and reps[-1].n == rows * C
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


@pytest.mark.parametrize("C", [1000, 32000, 40000])
@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
def test_subnormal_probabilities(gpu_lib, C, act):
    run_case(gpu_lib, 5, C, act, seed=220 + C, z=spread_rows(C, act, 220 + C))


def test_widest_rows_unaligned(gpu_lib):
    """One row of 268431360 bf16 classes (the widest the split backward takes:
    65535 column blocks of 4096) starting 2 bytes past a 16-byte boundary, so
    the one-element-per-load form runs with every column block of the launch.
    dlogits on sampled columns (every block's first and last column, the
    target, random ones) against the oracle run on the whole row."""
    C = 65535 * 4096
    t = np.array([C - 3], np.int32)
    print(f"\n[xent split widest] C={C}", flush=True)
    z = synth.normal((1, C), 2.0, "bf16", 911, synth.STREAM_X)
    zd = padded(z, "bf16", offset=1)
    z64 = synth.to_f64(z, "bf16")
    ref = xe.fwd_bwd(z64, t, 1.0)                 # one row: scale = dloss / rows = 1
    L32 = ref["row_lse"].astype(np.float32)
    dz = gpu_lib.vjp_softmax_xent_bwd(zd, torch.from_numpy(t).to(DEV), torch.from_numpy(L32).to(DEV),
                                      torch.ones(1, device=DEV))
    starts = np.arange(0, C, 4096)
    cols = np.unique(np.concatenate([starts, starts + 4095, t,
                                     np.random.default_rng(5).integers(0, C, 200000)]))
    got = to_host(dz, "bf16")[:, cols]
    del dz, zd
    S, F = _dz_tols_at(z64[:, cols], cols, t, ref["row_lse"], L32, 1.0)
    r = pointwise(got, ref["dz"][:, cols], "bf16", S=S, floor=F, name="dlogits(sampled)")
    print("   ", r, flush=True)
    assert r.ok, str(r)
