"""The documented fixed summation orders, replayed bit for bit on the host.

Every parameter gradient and the mean cross-entropy are sums whose order
include/libvjp.h documents (and which is independent of scheduling).  These
tests read the stage-1 partials back from the caller's workspace and replay
the documented stage-2 order in numpy float32 (every addition rounded to
fp32, as on the GPU), then require bitwise equality; for the scatter-add they
replay the per-row order (sorted positions; runs longer than 32 in chunks of
32, then the chunk sums in order).  Together with the oracle comparisons this
pins the exact result, not only its accuracy.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import DEV, to_host

pytestmark = pytest.mark.gpu
F32 = np.float32


def _wave_sum(v):
    """The DPP tree of one wave: neighbour swap, pair swap, half-row mirror, row
    mirror, then lanes (0 + 16) + (32 + 48)."""
    v = np.asarray(v, F32).copy()
    i = np.arange(64)
    for perm in (i ^ 1, i ^ 2, (i & ~7) | (7 - (i & 7)), (i & ~15) | (15 - (i & 15))):
        v = (v + v[perm]).astype(F32)
    return F32(F32(v[0] + v[16]) + F32(v[32] + v[48]))


def _scalar_order(P):
    """1024 threads: thread r sums P[r], P[r + 1024], ... in order; wave trees;
    the sixteen wave sums in wave order."""
    P = np.asarray(P, F32)
    lane = np.zeros(1024, F32)
    for t in range(P.size):
        lane[t % 1024] = F32(lane[t % 1024] + P[t])
    waves = [_wave_sum(lane[64 * w:64 * w + 64]) for w in range(16)]
    s = waves[0]
    for w in waves[1:]:
        s = F32(s + w)
    return s


def _columns_order(P):
    """d >= 2: 128 row lanes each sum P[r][j], P[r + 128][j], ... in order, then the
    pairwise tree v[r] += v[r + s] for s = 64, ..., 1."""
    P = np.asarray(P, F32)
    T, d = P.shape
    v = np.zeros((128, d), F32)
    for t in range(T):
        v[t % 128] = (v[t % 128] + P[t]).astype(F32)
    s = 64
    while s >= 1:
        v[:s] = (v[:s] + v[s:2 * s]).astype(F32)
        s //= 2
    return v[0]


def test_weighted_sum_grad_w_order(gpu_lib):
    for n, d, acc in [(100000, 256, False), (50000, 7, True), (3000, 100, False)]:
        x = synth.to_torch(synth.normal((n, d), 1.0, "bf16", 600 + d, 0), "bf16", DEV).view(n, d)
        w = synth.to_torch(synth.normal((d,), 0.1, "bf16", 600 + d, 1), "bf16", DEV)
        dy = synth.to_torch(synth.normal((n,), 1.0, "bf16", 600 + d, 2), "bf16", DEV)
        ws = torch.empty(gpu_lib.vjp_weighted_sum_bwd_workspace_size(n, d) // 4, dtype=torch.float32, device=DEV)
        old = torch.randn(d, generator=torch.Generator().manual_seed(d)).to(DEV)
        dw = old.clone()
        gpu_lib.vjp_weighted_sum_bwd(dy, x, w, dw=dw, accumulate=acc, workspace=ws)
        P = to_host(ws, "f32").reshape(-1, d)
        want = _columns_order(P)
        if acc:
            want = (old.cpu().numpy().astype(F32) + want).astype(F32)
        assert np.array_equal(to_host(dw, "f32").view(np.uint32), want.view(np.uint32)), (n, d)


def test_scaled_silu_dw_order(gpu_lib):
    n = (1 << 20) + 777
    x = synth.to_torch(synth.normal((n,), 2.0, "f16", 610, 0), "f16", DEV)
    dy = synth.to_torch(synth.normal((n,), 1.0, "f16", 610, 2), "f16", DEV)
    w = torch.tensor([0.75], device=DEV)
    ws = torch.empty(gpu_lib.vjp_scaled_silu_bwd_workspace_size(n) // 4, dtype=torch.float32, device=DEV)
    _, dw = gpu_lib.vjp_scaled_silu_bwd(dy, x, w, workspace=ws)
    want = _scalar_order(to_host(ws, "f32"))
    assert to_host(dw, "f32").view(np.uint32)[0] == np.array([want], F32).view(np.uint32)[0]


def test_softmax_xent_mean_order(gpu_lib):
    rows, C = 5000, 300
    z = synth.to_torch(synth.normal((rows, C), 2.0, "bf16", 620, 0), "bf16", DEV).view(rows, C)
    t = torch.from_numpy(synth.targets(rows, C, 620)).to(DEV)
    ws = torch.empty(rows, dtype=torch.float32, device=DEV)
    out = gpu_lib.vjp_softmax_xent_fwd(z, t, workspace=ws)
    want = F32(_scalar_order(to_host(ws, "f32")) / F32(rows))
    assert to_host(out["loss"], "f32").view(np.uint32)[0] == np.array([want], F32).view(np.uint32)[0]


def test_layernorm_dw_db_order(gpu_lib):
    rows, cols = 3000, 200
    x = synth.to_torch(synth.normal((rows, cols), 1.0, "bf16", 630, 0), "bf16", DEV).view(rows, cols)
    dy = synth.to_torch(synth.normal((rows, cols), 1.0, "bf16", 630, 2), "bf16", DEV).view(rows, cols)
    w = torch.ones(cols, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(gpu_lib.vjp_layernorm_bwd_workspace_size(rows, cols) // 4, dtype=torch.float32, device=DEV)
    _, dw, db = gpu_lib.vjp_layernorm_bwd(dy, x, w, workspace=ws)
    P = to_host(ws, "f32").reshape(-1, 2 * cols)
    want = _columns_order(P)
    assert np.array_equal(to_host(dw, "f32").view(np.uint32), want[:cols].view(np.uint32))
    assert np.array_equal(to_host(db, "f32").view(np.uint32), want[cols:].view(np.uint32))


@pytest.mark.parametrize("M,V", [(6000, 500), (6000, 40000), (20000, 500)])
def test_scatter_add_row_order(gpu_lib, M, V):
    """Short runs (<= 32) summed in sorted order, long runs in 32-position
    chunks, on every plan path: M <= 16384 with keys below 2^15 (the counting
    plan), with a wider key range (radix passes), and M > 16384 (separate
    kernels)."""
    D = 40
    idx = synth.zipf_indices(M, V, 640)
    dy = synth.normal((M, D), 1.0, "bf16", 640, 2)
    dt, _ = gpu_lib.vjp_gather_rows_bwd(synth.to_torch(dy, "bf16", DEV).view(M, D),
                                        torch.from_numpy(idx).to(DEV), V)
    dy32 = synth.to_f64(dy, "bf16").astype(F32)
    order = oracle.gather.sorted_order(idx, V)
    want = np.zeros((V, D), F32)
    keys = idx[order]
    starts = np.flatnonzero(np.r_[True, keys[1:] != keys[:-1]])
    ends = np.r_[starts[1:], M]
    assert np.bincount(idx, minlength=V).max() > 32, "the case needs a long run"
    for a, b in zip(starts, ends):
        pos = order[a:b]
        if b - a <= 32:
            acc = np.zeros(D, F32)
            for p in pos:
                acc = (acc + dy32[p]).astype(F32)
        else:
            acc = np.zeros(D, F32)
            for c0 in range(0, b - a, 32):
                part = np.zeros(D, F32)
                for p in pos[c0:c0 + 32]:
                    part = (part + dy32[p]).astype(F32)
                acc = (acc + part).astype(F32)
        want[keys[a]] = acc
    assert np.array_equal(to_host(dt, "f32").view(np.uint32), want.view(np.uint32))
