"""Streams and graph capture.

The library launches only kernels, on the caller's stream, and allocates,
copies and clears nothing itself (outputs and workspaces are the caller's).
So a whole forward + backward step of every op can run on a side stream, or
be captured once in a HIP graph and replayed with new inputs copied into the
captured buffers.  Every op is deterministic, so each replay must equal the
eager results for the same inputs bit for bit.
"""
import pytest
import torch

import row_wise_backward_amd as rwb
import synth
from gpu_util import DEV

pytestmark = pytest.mark.gpu

BF16, F16, F32 = torch.bfloat16, torch.float16, torch.float32


class Step:
    """Static inputs, preallocated outputs and workspaces, and one step of
    every op (forward then backward) writing into them."""

    def __init__(self):
        e = lambda *shape, dtype=BF16: torch.empty(shape, dtype=dtype, device=DEV)
        self.inp = {
            "ws_x": e(2048, 256), "ws_w": e(256), "ws_dy": e(2048),
            "si_x": e(100003, dtype=F16), "si_w": e(1, dtype=F32), "si_dy": e(100003, dtype=F16),
            "sm_x": e(256, 1000), "sm_dy": e(256, 1000),
            "xe_z": e(128, 3000), "xe_t": e(128, dtype=torch.int32), "xe_dloss": e(1, dtype=F32),
            "ln_x": e(300, 700), "ln_w": e(700), "ln_b": e(700), "ln_dy": e(300, 700),
            "ga_tab": e(500, 96), "ga_idx": e(2000, dtype=torch.int32), "ga_dy": e(2000, 96),
        }
        f = lambda *shape, dtype=F32: torch.empty(shape, dtype=dtype, device=DEV)
        self.out = {
            "ws_y": e(2048), "ws_dx": e(2048, 256), "ws_dw": f(256),
            "si_y": e(100003, dtype=F16), "si_dx": e(100003, dtype=F16), "si_dw": f(1),
            "sm_y": e(256, 1000), "sm_dx": e(256, 1000), "sm_y2": e(256, 1000), "sm_lse": f(256),
            "sm_dx2": e(256, 1000),
            "xe_loss": f(1), "xe_max": f(128), "xe_lse": f(128), "xe_dz": e(128, 3000),
            "xe_ninv": f(1, dtype=torch.int32), "xe_loss2": f(1), "xe_lse2": f(128),
            "xe_dz2": e(128, 3000),
            "ln_y": e(300, 700), "ln_mean": f(300), "ln_rstd": f(300), "ln_dx": e(300, 700),
            "ln_dw": f(700), "ln_db": f(700),
            "rm_y": e(300, 700), "rm_rstd": f(300), "rm_dx": e(300, 700), "rm_dw": f(700),
            "ga_y": e(2000, 96), "ga_dt": f(500, 96), "ga_ninv": f(1, dtype=torch.int32),
        }
        b = lambda n: torch.empty(max(int(n), 1), dtype=torch.uint8, device=DEV)
        self.ws = {
            "ws": b(rwb.vjp_weighted_sum_bwd_workspace_size(2048, 256)),
            "si": b(rwb.vjp_scaled_silu_bwd_workspace_size(100003)),
            "xe": b(rwb.vjp_softmax_xent_workspace_size(128)),
            "xe2": b(rwb.vjp_softmax_xent_workspace_size(128)),
            "ln": b(rwb.vjp_layernorm_bwd_workspace_size(300, 700)),
            "rm": b(rwb.vjp_rmsnorm_bwd_workspace_size(300, 700)),
            "ga": b(rwb.vjp_gather_rows_bwd_workspace_size(2000, 500, 96)),
        }

    def load(self, seed):
        """Copy a seeded input set into the static input buffers (eager)."""
        for n, (k, t) in enumerate(self.inp.items()):
            if k == "xe_t":
                t.copy_(synth.targets_device(128, 3000, seed, DEV))
            elif k == "ga_idx":
                t.copy_(torch.from_numpy(synth.zipf_indices(2000, 500, seed)).to(DEV))
            elif k == "xe_dloss":
                t.fill_(0.5 + seed % 3)
            elif k == "si_w":
                t.fill_(0.75 - 0.25 * (seed % 2))
            else:
                sd = {torch.bfloat16: "bf16", torch.float16: "f16"}[t.dtype]
                t.copy_(synth.normal_device(tuple(t.shape), 2.0, sd, seed, n, DEV))

    def run(self):
        i, o, w = self.inp, self.out, self.ws
        rwb.vjp_weighted_sum_fwd(i["ws_x"], i["ws_w"], y=o["ws_y"])
        rwb.vjp_weighted_sum_bwd(i["ws_dy"], i["ws_x"], i["ws_w"], dx=o["ws_dx"], dw=o["ws_dw"],
                                 workspace=w["ws"])
        rwb.vjp_scaled_silu_fwd(i["si_x"], i["si_w"], y=o["si_y"])
        rwb.vjp_scaled_silu_bwd(i["si_dy"], i["si_x"], i["si_w"], dx=o["si_dx"], dw=o["si_dw"],
                                workspace=w["si"])
        rwb.vjp_softmax_fwd(i["sm_x"], y=o["sm_y"])
        rwb.vjp_softmax_bwd(i["sm_dy"], o["sm_y"], dx=o["sm_dx"])
        rwb.vjp_softmax_fwd_lse(i["sm_x"], y=o["sm_y2"], row_lse=o["sm_lse"])
        rwb.vjp_softmax_bwd_lse(i["sm_dy"], i["sm_x"], o["sm_lse"], dx=o["sm_dx2"])
        rwb.vjp_softmax_xent_fwd_bwd(i["xe_z"], i["xe_t"], dlogits=o["xe_dz"], loss=o["xe_loss"],
                                     row_max=o["xe_max"], row_lse=o["xe_lse"],
                                     n_invalid=o["xe_ninv"], workspace=w["xe"])
        rwb.vjp_softmax_xent_fwd(i["xe_z"], i["xe_t"], loss=o["xe_loss2"], row_lse=o["xe_lse2"],
                                 count_invalid=False, workspace=w["xe2"])
        rwb.vjp_softmax_xent_bwd(i["xe_z"], i["xe_t"], o["xe_lse2"], i["xe_dloss"],
                                 dlogits=o["xe_dz2"])
        rwb.vjp_layernorm_fwd(i["ln_x"], i["ln_w"], i["ln_b"], y=o["ln_y"], row_mean=o["ln_mean"],
                              row_rstd=o["ln_rstd"])
        rwb.vjp_layernorm_bwd(i["ln_dy"], i["ln_x"], i["ln_w"], o["ln_mean"], o["ln_rstd"],
                              dx=o["ln_dx"], dw=o["ln_dw"], db=o["ln_db"], workspace=w["ln"])
        rwb.vjp_rmsnorm_fwd(i["ln_x"], i["ln_w"], y=o["rm_y"], row_rstd=o["rm_rstd"])
        rwb.vjp_rmsnorm_bwd(i["ln_dy"], i["ln_x"], i["ln_w"], o["rm_rstd"], dx=o["rm_dx"],
                            dw=o["rm_dw"], workspace=w["rm"])
        rwb.vjp_gather_rows_fwd(i["ga_tab"], i["ga_idx"], y=o["ga_y"])
        rwb.vjp_gather_rows_bwd(i["ga_dy"], i["ga_idx"], 500, dtable=o["ga_dt"],
                                n_invalid=o["ga_ninv"], workspace=w["ga"])

    def snapshot(self):
        torch.cuda.synchronize()
        return {k: t.clone() for k, t in self.out.items()}


def _same(a, b):
    bad = [k for k in a if not torch.equal(a[k].view(torch.uint8), b[k].view(torch.uint8))]
    assert not bad, f"outputs differ bitwise: {bad}"


def test_side_stream_matches_default_stream(gpu_lib):
    st = Step()
    st.load(11)
    st.run()
    ref = st.snapshot()
    for k in st.out:
        st.out[k].fill_(0)
    side = torch.cuda.Stream()   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    side.synchronize()
    _same(ref, st.snapshot())


def test_two_streams_at_once(gpu_lib):
    """Two steps with their own buffers and inputs, launched on two streams
    with nothing ordering them: calls share no state (each has its own
    workspace), so each step equals its own eager result bit for bit."""
    a, b = Step(), Step()
    a.load(31)
    a.run()
    ref_a = a.snapshot()
    b.load(32)
    b.run()
    ref_b = b.snapshot()
    for st in (a, b):
        for k in st.out:
            st.out[k].fill_(0)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(sa):
            a.run()
        with torch.cuda.stream(sb):
            b.run()
    torch.cuda.synchronize()
    _same(ref_a, a.snapshot())
    _same(ref_b, b.snapshot())


def test_graph_capture_replays_bitwise(gpu_lib):
    st = Step()
    refs = {}
    for seed in (21, 22):
        st.load(seed)
        st.run()
        refs[seed] = st.snapshot()
    assert not torch.equal(refs[21]["xe_dz"], refs[22]["xe_dz"])
    # warm up on a side stream, then capture one step
    st.load(21)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()
    for rep, seed in enumerate((22, 21, 22, 21)):
        st.load(seed)                    # eager copies into the captured inputs
        for k in st.out:                 # eager work between replays
            st.out[k].fill_(1 + rep)
        graph.replay()
        _same(refs[seed], st.snapshot())


@pytest.mark.parametrize("V", [40000, 32000])
def test_graph_scatter_add_zero_rows_across_launches(gpu_lib, V):
    """A V x 2048 fp32 gradient table (up to 328 MB): its never-selected rows
    are zero-filled partly beside the plan launches (three radix launches for
    40000 rows, the one counting launch for 32000) and partly by the
    listed-rows kernel.  Captured once, replayed with new indices and dy (the
    table poisoned between replays), every replay equals the eager result bit
    for bit."""
    print(f"\n[graph scatter-add] V={V}", flush=True)
    M, D = 6000, 2048
    idx = torch.empty(M, dtype=torch.int32, device=DEV)
    dy = torch.empty((M, D), dtype=BF16, device=DEV)
    dt = torch.empty((V, D), dtype=F32, device=DEV)
    ninv = torch.empty(1, dtype=torch.int32, device=DEV)
    ws = torch.empty(gpu_lib.vjp_gather_rows_bwd_workspace_size(M, V, D), dtype=torch.uint8,
                     device=DEV)

    def load(seed):
        idx.copy_(torch.from_numpy(synth.zipf_indices(M, V, seed)).to(DEV))
        dy.copy_(synth.normal_device((M, D), 1.0, "bf16", seed, 0, DEV))

    def run():
        gpu_lib.vjp_gather_rows_bwd(dy, idx, V, dtable=dt, n_invalid=ninv, workspace=ws)

    refs = {}
    for seed in (31, 32):
        load(seed)
        dt.fill_(float("nan"))
        run()
        torch.cuda.synchronize()
        refs[seed] = dt.clone()
        assert not torch.isnan(refs[seed]).any()
    load(31)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for seed in (32, 31, 32):
        load(seed)
        dt.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dt.view(torch.int32), refs[seed].view(torch.int32)), seed
