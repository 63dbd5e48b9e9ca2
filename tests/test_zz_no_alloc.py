"""The no-allocation scaled-SiLU backward against the workspace entry point.

vjp_scaled_silu_bwd_noalloc keeps its stage-1 partials in the library's
per-GPU scratch instead of a caller workspace; its kernels and summation
order are those of vjp_scaled_silu_bwd, so dx and dw must match it bit for
bit.  Two calls in a row, the second on a smaller input (the scratch keeps
the first call's partials past the second call's tiles), then one that
accumulates; plus the argument errors."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu
VJP_EINVAL, VJP_EDTYPE = 1, 2          # include/libvjp.h


def _inputs(n, act, seed):
    x = synth.to_torch(synth.normal((n,), 2.0, act, seed, synth.STREAM_X), act, DEV)
    dy = synth.to_torch(synth.normal((n,), 1.0, act, seed, synth.STREAM_DY), act, DEV)
    return x, dy


def _both(rwb, n, act, seed, accumulate=False):
    print(f"\n[no-alloc scaled_silu_bwd] n={n} act={act} accumulate={accumulate}", flush=True)
    x, dy = _inputs(n, act, seed)
    w = torch.tensor([0.75], dtype=torch.float32, device=DEV)
    old = torch.tensor([2.5], dtype=torch.float32, device=DEV)
    dx_ref = torch.full_like(x, float("nan"))
    dw_ref = old.clone() if accumulate else torch.full((1,), float("nan"), device=DEV)
    rwb.vjp_scaled_silu_bwd(dy, x, w, dx=dx_ref, dw=dw_ref, accumulate=accumulate)
    dx = torch.full_like(x, float("nan"))
    dw = old.clone() if accumulate else torch.full((1,), float("nan"), device=DEV)
    rwb.vjp_scaled_silu_bwd_noalloc(dy, x, w, dx, dw, accumulate=accumulate)
    torch.cuda.synchronize()
    same_dx = torch.equal(dx.view(torch.int16 if dx.element_size() == 2 else torch.int32),
                          dx_ref.view(torch.int16 if dx.element_size() == 2 else torch.int32))
    same_dw = torch.equal(dw.view(torch.int32), dw_ref.view(torch.int32))
    print(f"    dx bitwise equal: {same_dx}; dw {dw.item()!r} vs {dw_ref.item()!r}", flush=True)
    assert same_dx and same_dw


def test_two_calls_second_smaller(gpu_lib):
    _both(gpu_lib, 1 << 24, "f16", 1001)          # 4096 tiles: the whole scratch
    _both(gpu_lib, 100003, "f16", 1002)           # 49 tiles
    _both(gpu_lib, 7, "bf16", 1003)               # one tile, no vector loads
    _both(gpu_lib, 8193, "f32", 1004, accumulate=True)


def test_empty_and_errors(gpu_lib):
    x = torch.empty(0, dtype=torch.float16, device=DEV)
    w = torch.tensor([0.75], device=DEV)
    dw = torch.full((1,), 3.0, device=DEV)
    gpu_lib.vjp_scaled_silu_bwd_noalloc(x, x, w, x, dw)
    torch.cuda.synchronize()
    assert dw.item() == 0.0
    L = gpu_lib.lib
    y = torch.zeros(64, dtype=torch.float16, device=DEV)
    P = lambda t: t.data_ptr()  # noqa: E731
    assert L.vjp_scaled_silu_bwd_noalloc(P(y), P(y), P(w), P(y), P(dw), 0, 64, 7, None) == VJP_EDTYPE
    assert L.vjp_scaled_silu_bwd_noalloc(P(y), P(y), P(w), P(y), P(dw), 2, 64, 1, None) == VJP_EINVAL
    assert L.vjp_scaled_silu_bwd_noalloc(P(y), P(y), P(w), P(y), P(dw), 0, -1, 1, None) == VJP_EINVAL


def test_graph_capture_replays(gpu_lib):
    """The caller the entry point is for: a backward captured once in a HIP
    graph (nothing to allocate inside the capture) and replayed with new
    inputs copied into the captured buffers, eager work between the replays;
    every replay equals the workspace entry point bit for bit."""
    n, act = 100003, "f16"
    print(f"\n[no-alloc scaled_silu_bwd graph] n={n} act={act}", flush=True)
    x, dy = _inputs(n, act, 2001)
    w = torch.tensor([0.75], dtype=torch.float32, device=DEV)
    dx = torch.empty_like(x)
    dw = torch.empty(1, dtype=torch.float32, device=DEV)
    gpu_lib.vjp_scaled_silu_bwd_noalloc(dy, x, w, dx, dw)     # first call on the device: set-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu_lib.vjp_scaled_silu_bwd_noalloc(dy, x, w, dx, dw)
    torch.cuda.synchronize()
    for rep, seed in enumerate((2002, 2003, 2002)):
        xs, dys = _inputs(n, act, seed)
        x.copy_(xs)
        dy.copy_(dys)
        dx.fill_(float("nan"))
        dw.fill_(float(rep))
        graph.replay()
        dx_ref, dw_ref = gpu_lib.vjp_scaled_silu_bwd(dys, xs, w)
        torch.cuda.synchronize()
        same_dx = torch.equal(dx.view(torch.int16), dx_ref.view(torch.int16))
        same_dw = torch.equal(dw.view(torch.int32), dw_ref.view(torch.int32))
        print(f"    replay {rep}: dx bitwise equal {same_dx}; dw {dw.item()!r} vs {dw_ref.item()!r}",
              flush=True)
        assert same_dx and same_dw
