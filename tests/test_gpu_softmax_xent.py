"""Fused softmax-cross-entropy on the GPU vs the CPU oracle (calls the C ABI).

Tolerances: row_max bitwise (it is one of the inputs); row_lse and the row
losses 1e-5 * max(|o|, |m| + |log l| + |z_t|); dlogits 2 ulp (16-bit) or
1e-5 * max(|o|, grad_scale (p + [j = t])) (fp32), with a floor of
16 u grad_scale for the target entry p - 1; the mean loss 1e-4 relative;
n_invalid exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, Guarded, chunked, empty_padded, padded, to_host
from oracle.compare import U32, combine, exact, pointwise, reduced
from synth.workloads import XENT

pytestmark = pytest.mark.gpu
xe = oracle.softmax_xent


def _compare(out_gpu, z64, t, scale, act, rows_idx=None, ws_rows=None, name="xent"):
    ref = xe.fwd_bwd(z64, t, scale)
    reps = []
    m, lse = ref["row_max"], ref["row_lse"]
    zt = np.where((t >= 0) & (t < z64.shape[1]), z64[np.arange(len(t)), np.clip(t, 0, z64.shape[1] - 1)], 0)
    S_lse = np.abs(m) + np.abs(lse - m)
    reps.append(exact(out_gpu["row_max"], m.astype(np.float32), "f32", name="row_max"))
    reps.append(pointwise(out_gpu["row_lse"], lse, "f32", S=S_lse, name="row_lse"))
    if ws_rows is not None:
        reps.append(pointwise(ws_rows, ref["row_loss"], "f32", S=S_lse + np.abs(zt), name="row_loss"))
    p = np.exp(z64 - lse[:, None])
    onehot = np.zeros_like(p)
    valid = (t >= 0) & (t < z64.shape[1])
    onehot[np.arange(len(t))[valid], t[valid]] = 1.0
    S_dz = np.abs(scale) * (p + np.abs(onehot))
    F = 16 * U32 * np.abs(scale) * np.abs(onehot)
    reps.append(pointwise(out_gpu["dlogits"], ref["dz"], act, S=S_dz, floor=F, name="dlogits"))
    return ref, reps


def run_case(rwb, rows, C, act, seed, sigma=2.0, ld=None, offset=0, targets=None, scale=None,
             z=None):
    print(f"\n[softmax_xent] rows={rows} C={C} act={act} ld={ld} off={offset}", flush=True)
    if z is None:
        z = synth.normal((rows, C), sigma, act, seed, synth.STREAM_X)
    t = synth.targets(rows, C, seed) if targets is None else np.asarray(targets, np.int32)
    z64 = synth.to_f64(z, act)
    scale = 1.0 / rows if scale is None else scale
    zd = padded(z, act, ld, offset)
    td = torch.from_numpy(t).to(DEV)
    dz, dzbuf = empty_padded(rows, C, act, ld, offset)
    loss = Guarded(1, torch.float32)
    rmax = Guarded(rows, torch.float32)
    rlse = Guarded(rows, torch.float32)
    ninv = Guarded(1, torch.int32)
    wsg = Guarded(rwb.vjp_softmax_xent_workspace_size(rows) // 4, torch.float32)
    rwb.vjp_softmax_xent_fwd_bwd(zd, td, grad_scale=scale, dlogits=dz, loss=loss.t, row_max=rmax.t,
                                 row_lse=rlse.t, n_invalid=ninv.t, workspace=wsg.t)
    torch.cuda.synchronize()
    assert loss.intact() and rmax.intact() and rlse.intact() and ninv.intact() and wsg.intact()
    out = {"row_max": to_host(rmax.t, "f32"), "row_lse": to_host(rlse.t, "f32"),
           "dlogits": to_host(dz, act)}
    ref, reps = _compare(out, z64, t, scale, act, ws_rows=to_host(wsg.t, "f32"))
    reps.append(reduced(to_host(loss.t, "f32"), np.array([ref["loss"]]), name="loss"))
    n_inv = int(ninv.t.item())
    assert n_inv == ref["n_invalid"], (n_inv, ref["n_invalid"])
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
    run_case(gpu_lib, 7 if C > 4096 else 37, C, act, seed=90 + C)


@pytest.mark.parametrize("C", [1, 7, 2048, 16384, 17000])
def test_classes_f32(gpu_lib, C):
    run_case(gpu_lib, 7, C, "f32", seed=95 + C)


@pytest.mark.parametrize("C", [7, 32000, 40000])
@pytest.mark.parametrize("layout", ["padded_ld", "unaligned"])
def test_layouts(gpu_lib, C, layout):
    ld, off = (C + 8, 0) if layout == "padded_ld" else (C + 1, 1)
    run_case(gpu_lib, 5, C, "bf16", seed=97 + C, ld=ld, offset=off)


def test_invalid_targets(gpu_lib):
    """Targets outside [0, C): NaN row loss and mean, no one-hot term, counted exactly."""
    run_case(gpu_lib, 6, 300, "bf16", seed=98, targets=[3, -1, 300, 0, 299, 2 ** 31 - 1])


@pytest.mark.parametrize("act,C", [("bf16", 300), ("f16", 300), ("f32", 301)])
def test_invalid_target_in_last_vector_padding(gpu_lib, act, C):
    """Rows padded to 304 elements take the vector path with C not a multiple of
    the vector width: targets C and 303 fall in the last vector's padding.  They
    are the only invalid targets, so the row losses and the mean must be NaN."""
    run_case(gpu_lib, 4, C, act, seed=96, ld=304, targets=[3, C, 0, 303])


def test_batch1_and_batch7(gpu_lib):
    run_case(gpu_lib, 1, 32000, "bf16", seed=99)
    run_case(gpu_lib, 7, 32000, "bf16", seed=99)


def test_uniform_and_dominant(gpu_lib):
    """Uniform logits (loss = log C) and one dominant logit per row (p_t -> 1)."""
    rows, C = 4, 32000
    z = np.zeros((rows, C), np.float32)
    z[2, 5] = 60.0
    z[3, 77] = 30.0
    zs = synth.f32_to_storage(z, "bf16")
    t = np.array([0, 31999, 5, 77], np.int32)
    out = gpu_lib.vjp_softmax_xent_fwd_bwd(padded(zs, "bf16"), torch.from_numpy(t).to(DEV))
    torch.cuda.synchronize()
    res = {"row_max": to_host(out["row_max"], "f32"), "row_lse": to_host(out["row_lse"], "f32"),
           "dlogits": to_host(out["dlogits"], "bf16")}
    ref, reps = _compare(res, synth.to_f64(zs, "bf16"), t, 1.0 / rows, "bf16")
    reps.append(reduced(to_host(out["loss"], "f32"), np.array([ref["loss"]]), name="loss"))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps)


def test_empty(gpu_lib):
    z = torch.empty((0, 10), dtype=torch.bfloat16, device=DEV)
    out = gpu_lib.vjp_softmax_xent_fwd_bwd(z, torch.empty(0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert np.isnan(out["loss"].item()) and out["n_invalid"].item() == 0


def test_full_size(gpu_lib):
    """The 16384 x 32000 bf16 workload in the benchmark's launch configuration:
    dlogits, row_max, row_lse and the row losses on every row (in chunks of
    512 rows), the mean loss over all rows (its condition number reported)."""
    c = XENT
    rows, C = c.shape
    print(f"\n[softmax_xent full] {rows}x{C}", flush=True)
    z = synth.normal((rows, C), c.sigma_x, c.dtype, c.seed, synth.STREAM_X)
    t = synth.targets(rows, C, c.seed)
    zd = padded(z, "bf16")
    dz, dzg = empty_padded(rows, C, "bf16")
    loss, rmax, rlse = Guarded(1, torch.float32), Guarded(rows, torch.float32), Guarded(rows, torch.float32)
    ninv = Guarded(1, torch.int32)
    wsg = Guarded(gpu_lib.vjp_softmax_xent_workspace_size(rows) // 4, torch.float32)
    gpu_lib.vjp_softmax_xent_fwd_bwd(zd, torch.from_numpy(t).to(DEV), grad_scale=c.extra["grad_scale"],
                                     dlogits=dz, loss=loss.t, row_max=rmax.t, row_lse=rlse.t,
                                     n_invalid=ninv.t, workspace=wsg.t)
    torch.cuda.synchronize()
    assert dzg.intact() and loss.intact() and rmax.intact() and rlse.intact() and ninv.intact() \
        and wsg.intact(), "write outside an output"
    del zd
    out = {"row_max": to_host(rmax.t, "f32"), "row_lse": to_host(rlse.t, "f32"),
           "dlogits": to_host(dz, "bf16"), "row_loss": to_host(wsg.t, "f32")}
    del dz
    row_loss = np.empty(rows)

    def part(i, j):
        res = {k: v[i:j] for k, v in out.items() if k != "row_loss"}
        ref, reps = _compare(res, synth.to_f64(z[i:j], "bf16"), t[i:j], c.extra["grad_scale"], "bf16",
                             ws_rows=out["row_loss"][i:j])
        row_loss[i:j] = ref["row_loss"]
        return reps

    per = {}
    for reps in chunked(part, rows, 512):
        for r in reps:
            per.setdefault(r.name, []).append(r)
    reps = [combine(v, f"{k}(all rows)") for k, v in per.items()]
    reps.append(reduced(to_host(loss.t, "f32"), np.array([np.sum(row_loss) / rows]), name="loss",
                        S=[np.sum(np.abs(row_loss)) / rows]))
    assert int(ninv.t.item()) == 0
    for r in reps:
        print("   ", r, flush=True)
    assert {r.name: r.n for r in reps}["dlogits(all rows)"] == rows * C
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


@pytest.mark.parametrize("C", [1000, 32000, 40000])
@pytest.mark.parametrize("act", ["f32", "bf16", "f16"])
def test_subnormal_probabilities(gpu_lib, C, act):
    run_case(gpu_lib, 5, C, act, seed=120 + C, z=spread_rows(C, act, 120 + C))
