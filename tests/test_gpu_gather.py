"""Row gather and its deterministic scatter-add backward on the GPU vs the CPU
oracle (calls the C ABI).

y is a copy: bit-exact.  The sorted keys and positions in the workspace are
integers: bit-exact against the oracle's stable order.  dtable rows are fp32
sums of dy rows: |g - o| <= 1e-5 * max(|o|, S), S = the sum of |dy| over the
row's contributions (the fp32 rule for sums); n_invalid exact; two calls are
bitwise identical.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, Guarded, empty_padded, padded, to_host
from oracle.compare import exact, pointwise
from synth.workloads import EMBED

pytestmark = pytest.mark.gpu
ga = oracle.gather


def _indices(M, V, seed, kind):
    g = np.random.default_rng(seed)
    if kind == "zipf":
        return synth.zipf_indices(M, V, seed)
    if kind == "uniform":
        return g.integers(0, max(V, 1), size=M).astype(np.int32)
    if kind == "one_row":                     # every position selects the same row
        return np.full(M, V // 2, np.int32)
    if kind == "invalid_mix":                 # about a quarter outside [0, V)
        i = g.integers(-V // 3 - 2, V + V // 3 + 2, size=M)
        return i.astype(np.int32)
    if kind == "distinct":                    # M <= V rows, each selected once
        return g.permutation(V)[:M].astype(np.int32)
    raise ValueError(kind)


def run_case(rwb, M, V, D, act, seed, kind="zipf", ld=None, offset=0, accumulate=False):
    print(f"\n[gather] M={M} V={V} D={D} act={act} idx={kind} ld={ld} off={offset} acc={accumulate}",
          flush=True)
    idx = _indices(M, V, seed, kind)
    x = synth.normal((V, D), 1.0, act, seed, synth.STREAM_X)
    dy = synth.normal((M, D), 1.0, act, seed, synth.STREAM_DY)
    idx_d = torch.from_numpy(idx).to(DEV)
    xd = padded(x, act, ld, offset)
    y, _ = empty_padded(M, D, act, ld, offset)
    rwb.vjp_gather_rows_fwd(xd, idx_d, y=y)
    y_ref = ga.fwd(synth.to_f64(x, act), idx)
    reps = [exact(to_host(y, act), synth.f32_to_storage(y_ref.astype(np.float32), act), act, name="y")]

    dyd = padded(dy, act, ld, offset)
    old = np.random.default_rng(seed + 1).standard_normal((V, D)).astype(np.float32)
    dt, _ = empty_padded(V, D, "f32")
    if accumulate and V and D:
        dt.copy_(torch.from_numpy(old).to(DEV))
    need = rwb.vjp_gather_rows_bwd_workspace_size(M, V, D)
    wsg = Guarded(max(need // 4, 1), torch.float32)
    ninv = Guarded(1, torch.int32)
    rwb.vjp_gather_rows_bwd(dyd, idx_d, V, dtable=dt, accumulate=accumulate, n_invalid=ninv.t,
                            workspace=wsg.t)
    torch.cuda.synchronize()
    assert wsg.intact() and ninv.intact(), "write outside the workspace or count"
    dy64 = synth.to_f64(dy, act)
    dt_ref, n_inv = ga.bwd(dy64, idx, V, dx_old=old.astype(np.float64) if accumulate else None)
    S, _ = ga.bwd(np.abs(dy64), idx, V, dx_old=np.abs(old.astype(np.float64)) if accumulate else None)
    reps.append(pointwise(to_host(dt, "f32"), dt_ref, "f32", S=S, name="dtable"))
    assert int(ninv.t.item()) == n_inv, (int(ninv.t.item()), n_inv)
    if M > 0:
        wsi = wsg.t.view(torch.int32)
        order = ga.sorted_order(idx, V)
        keys = np.where(ga.valid_mask(idx, V), idx, V)[order].astype(np.int32)
        reps.append(exact(wsi[:M].cpu().numpy().view(np.float32), keys.view(np.float32), "f32",
                          name="sorted_keys"))
        reps.append(exact(wsi[M:2 * M].cpu().numpy().view(np.float32),
                          order.astype(np.int32).view(np.float32), "f32", name="sorted_positions"))
    for r in reps:
        print("   ", r, flush=True)
    assert all(r.ok for r in reps), [str(r) for r in reps if not r.ok]


# M <= 16384 builds the sort and run plan in one launch (V + 1 <= 32768: a
# counting sort) or three (a wider key range: radix passes), larger M with
# separate kernels: every side of both boundaries is covered.
CASES = [(1, 1, 1), (7, 5, 3), (1000, 37, 64), (2048, 300, 2049), (5000, 32000, 100),
         (3000, 70000, 40), (4097, 1, 16), (16384, 3000, 48), (16385, 3000, 48),
         (40000, 70000, 24), (50, 20, 70001),
         # the single-launch counting plan takes keys 0 .. V with V + 1 <= 32768
         (3000, 32767, 16), (3000, 32768, 16), (16384, 32767, 8)]


@pytest.mark.parametrize("M,V,D", CASES)
@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_shapes(gpu_lib, M, V, D, act):
    run_case(gpu_lib, M, V, D, act, seed=500 + M + V + D)


@pytest.mark.parametrize("kind", ["uniform", "one_row", "invalid_mix"])
def test_index_patterns(gpu_lib, kind):
    run_case(gpu_lib, 3000, 257, 130, "bf16", seed=510, kind=kind)


@pytest.mark.parametrize("kind", ["one_row", "distinct", "invalid_mix"])
def test_counting_plan_extremes(gpu_lib, kind):
    """The single-launch counting plan at its largest M (16384): one row
    selected by every index (its count at the top of the 16-bit fields), every
    index a different row (16384 listed rows, so the list of run starts takes
    all M + 1 entries), and a quarter of the indices invalid."""
    run_case(gpu_lib, 16384, 32767, 16, "bf16", seed=517, kind=kind)


def test_long_runs_and_accumulate(gpu_lib):
    """One row selected 5000 times (157 chunks of 32), accumulated into an
    existing gradient."""
    run_case(gpu_lib, 5000, 64, 300, "f16", seed=511, kind="one_row", accumulate=True)


@pytest.mark.parametrize("layout", ["padded_ld", "unaligned"])
def test_layouts(gpu_lib, layout):
    D = 100
    ld, off = (D + 8, 0) if layout == "padded_ld" else (D + 1, 1)
    run_case(gpu_lib, 700, 90, D, "bf16", seed=512, ld=ld, offset=off)


def test_batch1_and_batch7(gpu_lib):
    run_case(gpu_lib, 1, 10, 64, "bf16", seed=513)
    run_case(gpu_lib, 7, 3, 64, "bf16", seed=513, kind="uniform")


def test_empty(gpu_lib):
    dy = torch.empty((0, 8), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty(0, dtype=torch.int32, device=DEV)
    dt, n = gpu_lib.vjp_gather_rows_bwd(dy, idx, 5)
    torch.cuda.synchronize()
    assert bool((dt == 0).all()) and int(n.item()) == 0
    dt2, n2 = gpu_lib.vjp_gather_rows_bwd(torch.ones((3, 8), dtype=torch.bfloat16, device=DEV),
                                          torch.tensor([0, 1, 2], dtype=torch.int32, device=DEV), 0)
    torch.cuda.synchronize()
    assert dt2.shape == (0, 8) and int(n2.item()) == 3


def test_deterministic(gpu_lib):
    idx = torch.from_numpy(synth.zipf_indices(20000, 5000, 514)).to(DEV)
    dy = synth.to_torch(synth.normal((20000, 256), 1.0, "bf16", 514, 2), "bf16", DEV).view(20000, 256)
    a, _ = gpu_lib.vjp_gather_rows_bwd(dy, idx, 5000)
    b, _ = gpu_lib.vjp_gather_rows_bwd(dy, idx, 5000)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_zero_rows_across_every_launch(gpu_lib):
    """A 70000 x 2048 fp32 gradient table (573 MB; three radix passes): its
    never-selected rows are zero-filled partly beside each plan launch and
    partly by the listed-rows kernel.  The table starts as NaN, so a row
    that no launch writes fails the comparison."""
    run_case(gpu_lib, 16384, 70000, 2048, "bf16", seed=515, kind="uniform")


def test_full_size(gpu_lib):
    """16384 Zipf(1.2) token ids over a 32000 x 4096 bf16 table: y and every
    gradient row against the oracle."""
    c = EMBED
    M, D = c.shape
    V = c.extra["V"]
    print(f"\n[gather full] M={M} V={V} D={D}", flush=True)
    idx = synth.zipf_indices(M, V, c.seed, c.extra["zipf_a"])
    idx_d = torch.from_numpy(idx).to(DEV)
    x = synth.normal((V, D), c.sigma_x, "bf16", c.seed, synth.STREAM_X)
    y = gpu_lib.vjp_gather_rows_fwd(synth.to_torch(x, "bf16", DEV).view(V, D), idx_d)
    y_ref = ga.fwd(synth.to_f64(x, "bf16"), idx)
    ry = exact(to_host(y, "bf16"), synth.f32_to_storage(y_ref.astype(np.float32), "bf16"), "bf16",
               name="y")
    print("   ", ry, flush=True)
    del x, y, y_ref
    dy = synth.normal((M, D), 1.0, "bf16", c.seed, synth.STREAM_DY)
    dt, n = gpu_lib.vjp_gather_rows_bwd(synth.to_torch(dy, "bf16", DEV).view(M, D), idx_d, V)
    torch.cuda.synchronize()
    dy64 = synth.to_f64(dy, "bf16")
    dt_ref, n_inv = ga.bwd(dy64, idx, V)
    S, _ = ga.bwd(np.abs(dy64), idx, V)
    r = pointwise(to_host(dt, "f32"), dt_ref, "f32", S=S, name="dtable")
    print("   ", r, flush=True)
    assert ry.ok and r.ok and int(n.item()) == n_inv == 0


def test_widest_rows_unaligned(gpu_lib):
    """D = 16776960, the widest the gather and scatter-add take: 65535 column
    blocks of 256 in the one-element-per-load form (rows 2 bytes past a
    16-byte boundary), forward and backward."""
    run_case(gpu_lib, 3, 2, 65535 * 256, "bf16", 978, kind="uniform", offset=1)
