#!/usr/bin/env python3
"""Throughput of the VJP hot path on one MI355X.

One step is one forward and one backward of every op at its large workload,
in autograd order (all forwards, then the backwards in reverse):

  weighted_sum fwd   x bf16 [1048576, 256], w bf16 [256]
  scaled_silu fwd    x fp16 [2^24], w fp32 = 0.75
  softmax fwd        x bf16 [32768, 4096]
  softmax_xent       logits bf16 [16384, 32000] (fused forward + backward)
  softmax bwd        dy, y bf16 [32768, 4096]
  scaled_silu bwd    dy, x fp16 [2^24]         (+ fixed-order dw reduction)
  weighted_sum bwd   dy bf16 [1048576], x      (+ fixed-order grad_w reduction)

Every input is synthetic, seeded and already resident in HBM when timing
starts.  `value` is the step's algorithmic HBM bytes (what each kernel must
read and write once) divided by the measured step time over K warm steps
whose only instrumentation is one pair of HIP events around the `roofline`
op (the op with the largest share of the step), on the stream the kernels
are launched on; its `achieved` comes from those events.

`pairs_cold` (the primary per-pair figures) follow the flushed protocol:
before every launch group (one op: its kernels, stage 2 included; or one
copy), 1 GiB of plain stores evicts L2 and the 256 MB Infinity Cache; each
group runs 3 + 20 times and the median of the last 20 is kept.  By default
the protocol runs in a child process under `rocprofv3 --kernel-trace`
(started before this process uses the GPU) and a group's time is the sum of
its kernel durations; if that fails, or this process already runs under a
profiler, HIP events around each group in this process stand in (the line
says which).  The protocol also sweeps the launch shapes of the library's
streaming copy over the largest op's bytes (`copy_ceiling`: the best of
them) and copies each op's own byte count (`frac_of_matched_copy`).
`per_op` / `pairs` are the warm step's ops (a separate pass with events
around every op); `extras` / `extra_pairs_cold` cover the widened rows
(softmax saving the logsumexp, split cross-entropy, LayerNorm / RMSNorm on
[32768, 4096] bf16, the embedding gather with its deterministic scatter-add
backward over 16384 Zipf ids into a 32000 x 4096 table).  `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workloads, on all
cores and on one.  After timing, the outputs of every op are checked on the
GPU (`checks`: invariants and fp32 recomputations of sampled rows, each as
worst error / bound); a failed check ends the run with status 1 and no line.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fwd+bwd achieved HBM GB/s and % of MI355X peak; elements/s per op"
PEAK_GBS = 8000.0          # MI355X HBM3E, published
# Forward + backward pairs of the step (the fused cross-entropy is its own pair).
PAIRS = [("weighted_sum", ("weighted_sum_fwd", "weighted_sum_bwd")),
         ("scaled_silu", ("scaled_silu_fwd", "scaled_silu_bwd")),
         ("softmax", ("softmax_fwd", "softmax_bwd")),
         ("softmax_xent", ("softmax_xent_fwd_bwd",))]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_softmax_xent_bf16_16384x32000.json")


# Sources that define the fused cross-entropy kernels (the op with the largest
# share of the step) and the device compile flags: stored counter readings for
# it expire when any of them changes.
XENT_SOURCES = ("softmax_xent.hip", "reduce.hip", "rowops.hpp", "common.hpp", "launch.hpp")


def _compile_flags() -> list:
    """The library's hipcc flags, include directories named without their
    location (the tree sits at different paths on different hosts)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_vjp_build", os.path.join(ROOT, "row_wise_backward_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return [os.path.basename(f) if os.path.isabs(f) else f for f in mod.compile_flags()]


def source_digest(files=XENT_SOURCES) -> str:
    """Hash of the named kernel sources and of the compile flags."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_wise_backward_amd", "csrc")
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    h.update(" ".join(_compile_flags()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- bytes
# Algorithmic HBM bytes per call: every input read once, every output written once,
# stage-1 partials written once and read once by stage 2.

def bytes_weighted_sum_fwd(n, d, es=2, ws=2):
    return n * d * es + d * ws + n * es


def bytes_weighted_sum_bwd(n, d, T, es=2, ws=2):
    return n * es + n * d * es + d * ws + n * d * es + 2 * T * d * 4 + d * 4


def bytes_silu_fwd(n, es=2):
    return 2 * n * es + 4


def bytes_silu_bwd(n, T, es=2):
    return 3 * n * es + 4 + 2 * T * 4 + 4


def bytes_softmax_fwd(r, c, es=2):
    return 2 * r * c * es


def bytes_softmax_bwd(r, c, es=2):
    return 3 * r * c * es


def bytes_xent(r, c, es=2):
    # logits read, dlogits written, targets read (main kernel and finalize),
    # row_max / row_lse written, row losses written then read, loss + count written
    return 2 * r * c * es + 2 * r * 4 + 2 * r * 4 + 2 * r * 4 + 8


def bytes_softmax_fwd_lse(r, c, es=2):
    return 2 * r * c * es + 4 * r


def bytes_softmax_bwd_lse(r, c, es=2):
    return 3 * r * c * es + 4 * r


def bytes_xent_fwd(r, c, es=2):
    # logits read once, targets read (main kernel and finalize), row_lse written,
    # row losses written then read, loss + count written
    return r * c * es + 2 * r * 4 + r * 4 + 2 * r * 4 + 8


def bytes_xent_bwd(r, c, es=2):
    # logits read, dlogits written, targets and row_lse read, dloss read
    return 2 * r * c * es + 2 * r * 4 + 4


def bytes_layernorm_fwd(r, c, es=2, ws=2):
    return 2 * r * c * es + 2 * c * ws + 8 * r


def bytes_layernorm_bwd(r, c, T, es=2, ws=2):
    return 3 * r * c * es + c * ws + 8 * r + 2 * T * 2 * c * 4 + 8 * c


def bytes_rmsnorm_fwd(r, c, es=2, ws=2):
    return 2 * r * c * es + c * ws + 4 * r


def bytes_rmsnorm_bwd(r, c, T, es=2, ws=2):
    return 3 * r * c * es + c * ws + 4 * r + 2 * T * c * 4 + 4 * c


def bytes_gather_fwd(M, D, es=2):
    # each output row reads its table row once; indices read
    return 2 * M * D * es + 4 * M


def bytes_gather_bwd(M, V, D, es=2):
    # dy read once, every fp32 gradient row written once, indices read
    return M * D * es + V * D * 4 + 4 * M


# ----------------------------------------------------------------------------- CPU baseline
# The fp64 CPU oracle timed on the host's cores.  The sample's inputs are
# drawn once and written to memory-mapped files; worker processes (started
# fresh, BLAS and OpenMP limited to one thread each) load them and run the
# oracle's forward and backward over chunks of rows or elements.  The
# chunking only spreads the work: every chunk calls the oracle functions as
# they are.  The one-core leg is the same with one worker.

_CPU = {}   # the memory-mapped sample, per worker process


def _cpu_worker_init(folder):
    import numpy as np

    for name in ("silu_x", "silu_g", "ws_x", "ws_w", "ws_g", "sm_x", "sm_g", "xe_z", "xe_t"):
        _CPU[name] = np.load(os.path.join(folder, name + ".npy"), mmap_mode="r")


def _cpu_task(task):
    """One chunk of the sample through the oracle: (op, lo, hi) rows or elements."""
    import oracle
    import synth

    op, lo, hi = task
    c = _CPU
    if op == "silu":
        x64, g64 = synth.to_f64(c["silu_x"][lo:hi], "f16"), synth.to_f64(c["silu_g"][lo:hi], "f16")
        oracle.scaled_silu.fwd(x64, 0.75)
        oracle.scaled_silu.bwd(g64, x64, 0.75)
    elif op == "ws":
        x64, w64 = synth.to_f64(c["ws_x"][lo:hi], "bf16"), synth.to_f64(c["ws_w"], "bf16")
        g64 = synth.to_f64(c["ws_g"][lo:hi], "bf16")
        oracle.weighted_sum.fwd(x64, w64)
        oracle.weighted_sum.bwd(g64, x64, w64)
    elif op == "softmax":
        y = oracle.softmax.fwd(synth.to_f64(c["sm_x"][lo:hi], "bf16"))
        oracle.softmax.bwd(synth.to_f64(c["sm_g"][lo:hi], "bf16"), y)
    elif op == "xent":
        oracle.softmax_xent.fwd_bwd(synth.to_f64(c["xe_z"][lo:hi], "bf16"),
                                    np_array(c["xe_t"][lo:hi]), 1.0 / 16384)
    return hi - lo


def np_array(a):
    import numpy as np

    return np.array(a)


def cpu_cores() -> int:
    """Cores this process may run on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(scale: float = 1.0, min_seconds: float = 10.0, cores: int | None = None):
    """The oracle (fp64 numpy) on a bounded sample of each workload: on all
    cores (one worker process per core) and on one core."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import numpy as np

    import synth

    n_silu = max(1 << 16, int((1 << 23) * scale))
    n_ws = max(1024, int(131072 * scale))
    r_sm = max(64, int(4096 * scale))
    r_xe = max(16, int(1024 * scale))
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    folder = tempfile.mkdtemp(prefix="vjp_oracle_", dir=shm)
    try:
        arrays = {
            "silu_x": synth.normal((n_silu,), 2.0, "f16", 1001, 0),
            "silu_g": synth.normal((n_silu,), 1.0, "f16", 1001, 2),
            "ws_x": synth.normal((n_ws, 256), 1.0, "bf16", 1002, 0),
            "ws_w": synth.normal((256,), 0.1, "bf16", 1002, 1),
            "ws_g": synth.normal((n_ws,), 1.0, "bf16", 1002, 2),
            "sm_x": synth.normal((r_sm, 4096), 3.0, "bf16", 1003, 0),
            "sm_g": synth.normal((r_sm, 4096), 1.0, "bf16", 1003, 2),
            "xe_z": synth.normal((r_xe, 32000), 2.0, "bf16", 1004, 0),
            "xe_t": synth.targets(r_xe, 32000, 1004),
        }
        for name, a in arrays.items():
            np.save(os.path.join(folder, name + ".npy"), a)
        del arrays
        sample_bytes = (bytes_silu_fwd(n_silu) + bytes_silu_bwd(n_silu, 1)
                        + bytes_weighted_sum_fwd(n_ws, 256) + bytes_weighted_sum_bwd(n_ws, 256, 1)
                        + bytes_softmax_fwd(r_sm, 4096) + bytes_softmax_bwd(r_sm, 4096)
                        + bytes_xent(r_xe, 32000))
        tasks = ([("silu", i, min(i + (1 << 19), n_silu)) for i in range(0, n_silu, 1 << 19)]
                 + [("ws", i, min(i + 8192, n_ws)) for i in range(0, n_ws, 8192)]
                 + [("softmax", i, min(i + 256, r_sm)) for i in range(0, r_sm, 256)]
                 + [("xent", i, min(i + 64, r_xe)) for i in range(0, r_xe, 64)])
        # big chunks first, so the last ones to finish are small
        tasks.sort(key=lambda t: -(t[2] - t[1]) * {"silu": 1, "ws": 256, "softmax": 4096,
                                                   "xent": 32000}[t[0]])

        def timed(n_workers):
            saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                                    "MKL_NUM_THREADS")}
            for k in saved:
                os.environ[k] = "1"
            try:
                ctx = mp.get_context("spawn")
                with ctx.Pool(n_workers, initializer=_cpu_worker_init, initargs=(folder,)) as pool:
                    # warm up (imports, file maps); every wait is bounded
                    pool.map_async(_cpu_task, [("silu", 0, 1)] * n_workers, chunksize=1).get(300)
                    reps = 0
                    t0 = time.perf_counter()
                    while True:
                        pool.map_async(_cpu_task, tasks, chunksize=1).get(600)
                        reps += 1
                        dt = time.perf_counter() - t0
                        if dt >= min_seconds:
                            break
            finally:
                for k, v in saved.items():
                    if v is None:
                        os.environ.pop(k, None)
                    else:
                        os.environ[k] = v
            return sample_bytes * reps / dt / 1e9, reps, dt

        n = cores or cpu_cores()
        v_all, reps_all, dt_all = timed(n)
        v_one, reps_one, dt_one = timed(1)
    finally:
        shutil.rmtree(folder, ignore_errors=True)
    sample = (f"fwd+bwd of scaled_silu n={n_silu}, weighted_sum {n_ws}x256, softmax {r_sm}x4096, "
              f"softmax_xent {r_xe}x32000 (the workloads' distributions and seeds; "
              f"{sample_bytes / 1e9:.3f} GB of algorithmic bytes: {scale:g} x 1/2, 1/8, 1/8 and "
              f"1/16 of the four workloads), fp64 numpy with input decode, in "
              f"{len(tasks)} chunks of rows or elements")
    return {
        "value": round(v_all, 4),
        "unit": "GB/s",
        "cores": n,
        "kind": "oracle",
        "sample": sample + f"; {n} worker processes, {reps_all} passes in {dt_all:.1f} s",
        "one_core": {"value": round(v_one, 4), "unit": "GB/s", "cores": 1,
                     "timing": f"one worker process, {reps_one} passes in {dt_one:.1f} s"},
    }


# ----------------------------------------------------------------------------- GPU

PROTOCOL_REPS, PROTOCOL_WARM = 20, 3
FLUSH_BYTES = 1 << 30
# Launch shapes of the copy sweep (16-byte vectors in flight per lane, grid bound).
COPY_SHAPES = [(vpl, wg) for vpl in (2, 4, 8) for wg in (8192, 16384, 32768, 65536)]
# Forward + backward pairs among the extras.
EXTRA_PAIRS = [("softmax_lse", ("softmax_fwd_lse", "softmax_bwd_lse")),
               ("softmax_xent_split", ("softmax_xent_fwd", "softmax_xent_bwd")),
               ("layernorm", ("layernorm_fwd", "layernorm_bwd")),
               ("rmsnorm", ("rmsnorm_fwd", "rmsnorm_bwd")),
               ("gather_rows", ("gather_rows_fwd", "gather_rows_bwd"))]


class Workbench:
    """Seeded inputs (drawn on the device), outputs, workspaces and the
    marshalled C calls of every op: ``ops`` are the step (all forwards, then
    the backwards in reverse), ``extra_ops`` the widened rows."""

    def __init__(self, dev):
        import torch

        import row_wise_backward_amd as rwb
        import synth
        from synth.workloads import EMBED, SILU_16M, SOFTMAX, WS_LARGE, XENT

        self.torch, self.rwb, self.L = torch, rwb, rwb.lib
        L = self.L
        e = lambda *a, **k: torch.empty(*a, device=dev, **k)  # noqa: E731
        bf, f32 = torch.bfloat16, torch.float32
        n_ws, d_ws = WS_LARGE.shape
        wx = synth.normal_device((n_ws, d_ws), WS_LARGE.sigma_x, "bf16", WS_LARGE.seed, 0, dev)
        ww = synth.normal_device((d_ws,), WS_LARGE.sigma_w, "bf16", WS_LARGE.seed, 1, dev)
        wg = synth.normal_device((n_ws,), WS_LARGE.sigma_dy, "bf16", WS_LARGE.seed, 2, dev)
        wy, wdx, wdw = e(n_ws, dtype=bf), torch.empty_like(wx), e(d_ws, dtype=f32)
        wws = e(rwb.vjp_weighted_sum_bwd_workspace_size(n_ws, d_ws), dtype=torch.uint8)
        T_ws = wws.numel() // (4 * d_ws)
        n_s = SILU_16M.shape[0]
        sx = synth.normal_device((n_s,), SILU_16M.sigma_x, "f16", SILU_16M.seed, 0, dev)
        sg = synth.normal_device((n_s,), SILU_16M.sigma_dy, "f16", SILU_16M.seed, 2, dev)
        sw = torch.tensor([SILU_16M.w_value], dtype=f32, device=dev)
        sy, sdx, sdw = torch.empty_like(sx), torch.empty_like(sx), e(1, dtype=f32)
        sws = e(rwb.vjp_scaled_silu_bwd_workspace_size(n_s), dtype=torch.uint8)
        T_s = sws.numel() // 4
        r_m, c_m = SOFTMAX.shape
        mx = synth.normal_device((r_m, c_m), SOFTMAX.sigma_x, "bf16", SOFTMAX.seed, 0, dev)
        mg = synth.normal_device((r_m, c_m), SOFTMAX.sigma_dy, "bf16", SOFTMAX.seed, 2, dev)
        my, mdx = torch.empty_like(mx), torch.empty_like(mx)
        r_x, c_x = XENT.shape
        z = synth.normal_device((r_x, c_x), XENT.sigma_x, "bf16", XENT.seed, 0, dev)
        tg = synth.targets_device(r_x, c_x, XENT.seed, dev)
        dz = torch.empty_like(z)
        loss, rmax, rlse = e(1, dtype=f32), e(r_x, dtype=f32), e(r_x, dtype=f32)
        ninv = e(1, dtype=torch.int32)
        xws = e(rwb.vjp_softmax_xent_workspace_size(r_x), dtype=torch.uint8)
        scale = XENT.extra["grad_scale"]

        # one checked pass through the binding (host-side shape guards) ...
        rwb.vjp_weighted_sum_fwd(wx, ww, y=wy)
        rwb.vjp_scaled_silu_fwd(sx, sw, y=sy)
        rwb.vjp_softmax_fwd(mx, y=my)
        rwb.vjp_softmax_xent_fwd_bwd(z, tg, grad_scale=scale, dlogits=dz, loss=loss, row_max=rmax,
                                     row_lse=rlse, n_invalid=ninv, workspace=xws)
        rwb.vjp_softmax_bwd(mg, my, dx=mdx)
        rwb.vjp_scaled_silu_bwd(sg, sx, sw, dx=sdx, dw=sdw, workspace=sws)
        rwb.vjp_weighted_sum_bwd(wg, wx, ww, dx=wdx, dw=wdw, workspace=wws)
        torch.cuda.synchronize()

        # ... then the same C calls with their arguments marshalled once
        P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
        self.P = P
        self.stream = stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        BF16, F16 = rwb.VJP_BF16, rwb.VJP_F16
        self.ops = [
            ("weighted_sum_fwd", L.vjp_weighted_sum_fwd,
             (P(wx), d_ws, P(ww), P(wy), n_ws, d_ws, BF16, BF16, stream),
             bytes_weighted_sum_fwd(n_ws, d_ws), n_ws * d_ws),
            ("scaled_silu_fwd", L.vjp_scaled_silu_fwd, (P(sx), P(sw), P(sy), n_s, F16, stream),
             bytes_silu_fwd(n_s), n_s),
            ("softmax_fwd", L.vjp_softmax_fwd, (P(mx), c_m, P(my), c_m, r_m, c_m, BF16, stream),
             bytes_softmax_fwd(r_m, c_m), r_m * c_m),
            ("softmax_xent_fwd_bwd", L.vjp_softmax_xent_fwd_bwd,
             (P(z), c_x, P(tg), r_x, c_x, BF16, ctypes.c_float(scale), P(loss), P(rmax), P(rlse), P(dz),
              c_x, P(ninv), P(xws), xws.numel(), stream),
             bytes_xent(r_x, c_x), r_x * c_x),
            ("softmax_bwd", L.vjp_softmax_bwd, (P(mg), c_m, P(my), c_m, P(mdx), c_m, r_m, c_m, BF16, stream),
             bytes_softmax_bwd(r_m, c_m), r_m * c_m),
            ("scaled_silu_bwd", L.vjp_scaled_silu_bwd,
             (P(sg), P(sx), P(sw), P(sdx), P(sdw), 0, n_s, F16, P(sws), sws.numel(), stream),
             bytes_silu_bwd(n_s, T_s), n_s),
            ("weighted_sum_bwd", L.vjp_weighted_sum_bwd,
             (P(wg), P(wx), d_ws, P(ww), P(wdx), d_ws, P(wdw), 0, n_ws, d_ws, 0, BF16, BF16, P(wws),
              wws.numel(), stream),
             bytes_weighted_sum_bwd(n_ws, d_ws, T_ws), n_ws * d_ws),
        ]

        # Widened rows: the statistics-saving softmax and split cross-entropy on
        # the same inputs, LayerNorm / RMSNorm on the softmax workload's shape,
        # the embedding gather and its scatter-add backward.
        mlse, dz2 = e(r_m, dtype=f32), torch.empty_like(z)
        dloss = torch.ones(1, dtype=f32, device=dev)
        nw = synth.normal_device((c_m,), 0.1, "bf16", SOFTMAX.seed, 1, dev) + 1.0
        nb = synth.normal_device((c_m,), 0.1, "bf16", SOFTMAX.seed, 3, dev)
        nmean, nrstd = e(r_m, dtype=f32), e(r_m, dtype=f32)
        ndw, ndb = e(c_m, dtype=f32), e(c_m, dtype=f32)
        lnws = e(rwb.vjp_layernorm_bwd_workspace_size(r_m, c_m), dtype=torch.uint8)
        rmsws = e(rwb.vjp_rmsnorm_bwd_workspace_size(r_m, c_m), dtype=torch.uint8)
        T_ln, T_rms = lnws.numel() // (8 * c_m), rmsws.numel() // (4 * c_m)
        F32 = ctypes.c_float
        e_M, e_D = EMBED.shape
        e_V = EMBED.extra["V"]
        e_idx = torch.from_numpy(synth.zipf_indices(e_M, e_V, EMBED.seed, EMBED.extra["zipf_a"])).to(dev)
        e_tab = synth.normal_device((e_V, e_D), 1.0, "bf16", EMBED.seed, 0, dev)
        e_y = e((e_M, e_D), dtype=bf)
        e_dy = synth.normal_device((e_M, e_D), 1.0, "bf16", EMBED.seed, 2, dev)
        e_dt = e((e_V, e_D), dtype=f32)
        e_ninv = e(1, dtype=torch.int32)
        e_ws = e(rwb.vjp_gather_rows_bwd_workspace_size(e_M, e_V, e_D), dtype=torch.uint8)
        self.extra_ops = [
            ("softmax_fwd_lse", L.vjp_softmax_fwd_lse,
             (P(mx), c_m, P(my), c_m, P(mlse), r_m, c_m, BF16, stream), bytes_softmax_fwd_lse(r_m, c_m),
             r_m * c_m),
            ("softmax_bwd_lse", L.vjp_softmax_bwd_lse,
             (P(mg), c_m, P(mx), c_m, P(mlse), P(mdx), c_m, r_m, c_m, BF16, stream),
             bytes_softmax_bwd_lse(r_m, c_m), r_m * c_m),
            ("softmax_xent_fwd", L.vjp_softmax_xent_fwd,
             (P(z), c_x, P(tg), r_x, c_x, BF16, P(loss), None, P(rlse), P(ninv), P(xws), xws.numel(),
              stream), bytes_xent_fwd(r_x, c_x), r_x * c_x),
            ("softmax_xent_bwd", L.vjp_softmax_xent_bwd,
             (P(z), c_x, P(tg), P(rlse), r_x, c_x, BF16, P(dloss), P(dz2), c_x, stream),
             bytes_xent_bwd(r_x, c_x), r_x * c_x),
            ("layernorm_fwd", L.vjp_layernorm_fwd,
             (P(mx), c_m, P(nw), P(nb), P(my), c_m, P(nmean), P(nrstd), r_m, c_m, F32(1e-5), BF16, BF16,
              stream), bytes_layernorm_fwd(r_m, c_m), r_m * c_m),
            ("layernorm_bwd", L.vjp_layernorm_bwd,
             (P(mg), c_m, P(mx), c_m, P(nw), P(nmean), P(nrstd), P(mdx), c_m, P(ndw), P(ndb), 0, r_m,
              c_m, F32(1e-5), BF16, BF16, P(lnws), lnws.numel(), stream),
             bytes_layernorm_bwd(r_m, c_m, T_ln), r_m * c_m),
            ("rmsnorm_fwd", L.vjp_rmsnorm_fwd,
             (P(mx), c_m, P(nw), P(my), c_m, P(nrstd), r_m, c_m, F32(1e-6), BF16, BF16, stream),
             bytes_rmsnorm_fwd(r_m, c_m), r_m * c_m),
            ("rmsnorm_bwd", L.vjp_rmsnorm_bwd,
             (P(mg), c_m, P(mx), c_m, P(nw), P(nrstd), P(mdx), c_m, P(ndw), 0, r_m, c_m, F32(1e-6),
              BF16, BF16, P(rmsws), rmsws.numel(), stream),
             bytes_rmsnorm_bwd(r_m, c_m, T_rms), r_m * c_m),
            ("gather_rows_fwd", L.vjp_gather_rows_fwd,
             (P(e_tab), e_D, e_V, e_D, P(e_idx), e_M, P(e_y), e_D, BF16, stream),
             bytes_gather_fwd(e_M, e_D), e_M * e_D),
            ("gather_rows_bwd", L.vjp_gather_rows_bwd,
             (P(e_dy), e_D, P(e_idx), e_M, e_V, e_D, P(e_dt), e_D, 0, P(e_ninv), BF16, P(e_ws),
              e_ws.numel(), stream),
             bytes_gather_bwd(e_M, e_V, e_D), e_M * e_D),
        ]
        self.keep = [v for v in locals().values() if isinstance(v, torch.Tensor)]
        self.t = {k: v for k, v in locals().items() if isinstance(v, torch.Tensor)}
        self.scale = scale
        # copy reference buffers: as many bytes as the largest op moves, half each way
        self.copy_half = max(o[3] for o in self.ops) // 32 * 16
        self.ca = e(self.copy_half, dtype=torch.uint8)
        self.cb = e(self.copy_half, dtype=torch.uint8)

    def call(self, op):
        name, fn, a = op[0], op[1], op[2]
        st = fn(*a)
        if st != 0:
            raise RuntimeError(f"{name}: status {st} ({self.rwb.vjp_last_error()})")

    def copy(self, nbytes, vpl=4, wg=32768, offset=0):
        """vjp_copy_shaped of nbytes (rounded down to 16) between the copy buffers."""
        n = min(nbytes // 16 * 16, self.copy_half)
        st = self.L.vjp_copy_shaped(ctypes.c_void_p(self.ca.data_ptr() + offset),
                                    ctypes.c_void_p(self.cb.data_ptr() + offset), n, vpl, wg,
                                    self.stream)
        if st != 0:
            raise RuntimeError(f"vjp_copy_shaped: status {st} ({self.rwb.vjp_last_error()})")
        return n


    # ------------------------------------------------------------- output checks
    # Sanity checks of what the timed launches computed, on the GPU with torch
    # in fp32: invariants of each result and recomputations of sampled rows.
    # They are not the parity tests (those compare every element with the CPU
    # oracle); they keep a launch that computes garbage from being reported
    # as a throughput.  Each check is (worst error / its bound): 1 or less
    # passes.  The bounds allow two units of the storage rounding (2^-7
    # relative for bf16, 2^-10 for fp16) plus the fp32 error of the values.

    def check_step(self):
        """The step's outputs, right after the timed steps."""
        torch, t = self.torch, self.t
        f = lambda a: a.float()  # noqa: E731
        worst = lambda err, bound: float((err / bound).max())  # noqa: E731
        out = {}
        # weighted sum: y and grad_x on every 257th row, grad_w against a GEMV
        rows = torch.arange(0, t["wx"].shape[0], 257, device=t["wx"].device)
        x, w, g = f(t["wx"][rows]), f(t["ww"]), f(t["wg"][rows])
        ref = (x * w).sum(1)
        out["weighted_sum_y"] = worst((f(t["wy"][rows]) - ref).abs(),
                                      2 ** -7 * ref.abs() + 1e-5 * (x * w).abs().sum(1) + 1e-30)
        exact = torch.equal(t["wdx"][rows], (g[:, None] * w).to(t["wdx"].dtype))
        out["weighted_sum_grad_x_exact"] = 0.0 if exact else float("inf")
        X, G = f(t["wx"]), f(t["wg"])
        dw_ref = torch.mv(X.t(), G)
        dw_abs = torch.mv(X.abs().t(), G.abs())
        del X
        out["weighted_sum_grad_w"] = worst((t["wdw"] - dw_ref).abs(), 1e-4 * dw_abs + 1e-30)
        # scaled SiLU: every element of y and dx, and dw
        x, g, wv = f(t["sx"]), f(t["sg"]), f(t["sw"])
        sg = torch.sigmoid(x)
        ref = wv * x * sg
        out["scaled_silu_y"] = worst((f(t["sy"]) - ref).abs(), 2 ** -10 * ref.abs() + 1e-7)
        ref = g * wv * (sg + x * sg * (1 - sg))
        out["scaled_silu_dx"] = worst((f(t["sdx"]) - ref).abs(),
                                      2 ** -10 * ref.abs() + 1e-4 * (g * wv).abs() * (1 + x.abs()) + 1e-7)
        terms = g * x * sg
        out["scaled_silu_dw"] = worst((t["sdw"] - terms.sum()).abs(), 1e-5 * terms.abs().sum() + 1e-30)
        # softmax: row sums of y and dx everywhere, every 129th row recomputed
        y, dy, dx = t["my"], t["mg"], t["mdx"]
        out["softmax_y_row_sums"] = float((f(y).sum(1) - 1).abs().max()) / 1e-2
        sdot = (f(dy) * f(y)).sum(1)
        out["softmax_dx_row_sums"] = worst(f(dx).sum(1).abs(), 1e-2 * (sdot.abs() + f(dx).abs().sum(1)) + 1e-30)
        rows = torch.arange(0, y.shape[0], 129, device=y.device)
        ref = torch.softmax(f(t["mx"][rows]), 1)
        out["softmax_y_rows"] = worst((f(y[rows]) - ref).abs(), 2 ** -7 * ref + 1e-30)
        ys, gs = f(y[rows]), f(dy[rows])
        ref = ys * (gs - sdot[rows, None])
        sabs = (gs.abs() * ys).sum(1, keepdim=True)
        out["softmax_dx_rows"] = worst((f(dx[rows]) - ref).abs(),
                                       2 ** -7 * ref.abs() + 1e-4 * ys * (gs.abs() + sabs) + 1e-30)
        out.update(self._check_xent(t["loss"], t["rlse"], t["dz"], self.scale, t["rmax"]))
        out["softmax_xent_n_invalid"] = 0.0 if int(t["ninv"].item()) == 0 else float("inf")
        return out

    def _check_xent(self, loss, lse, dz, scale, rmax=None, tag="softmax_xent"):
        torch, t = self.torch, self.t
        f = lambda a: a.float()  # noqa: E731
        worst = lambda err, bound: float((err / bound).max())  # noqa: E731
        z, tg = t["z"], t["tg"].long()
        R, C = z.shape
        ar = torch.arange(R, device=z.device)
        loss_ref = (lse - f(z[ar, tg])).mean()
        out = {f"{tag}_loss": float((loss - loss_ref).abs() / (1e-5 * loss_ref.abs() + 1e-30))}
        if rmax is not None:
            ok = bool((lse >= rmax).all()) and bool((lse <= rmax + float(torch.log(torch.tensor(float(C)))) + 1e-3).all())
            out[f"{tag}_lse_bounds"] = 0.0 if ok else float("inf")
        sums = torch.cat([f(dz[r:r + 1024]).sum(1) for r in range(0, R, 1024)])
        out[f"{tag}_dlogits_row_sums"] = float(sums.abs().max()) / (2e-2 * scale)
        rows = ar[::64]
        p = torch.exp(f(z[rows]) - lse[rows, None])
        p[torch.arange(rows.numel(), device=z.device), tg[rows]] -= 1.0
        ref = scale * p
        out[f"{tag}_dlogits_rows"] = worst((f(dz[rows]) - ref).abs(), 2 ** -7 * ref.abs() + 1e-6 * scale)
        return out

    def check_extras(self):
        """The widened rows: each op run once more, its outputs checked before
        the next op reuses the buffers."""
        torch, t = self.torch, self.t
        F = torch.nn.functional
        f = lambda a: a.float()  # noqa: E731
        worst = lambda err, bound: float((err / bound).max())  # noqa: E731
        ops = {o[0]: o for o in self.extra_ops}
        out = {}
        x, dy = t["mx"], t["mg"]
        rows = torch.arange(0, x.shape[0], 129, device=x.device)
        xs, gs = f(x[rows]), f(dy[rows])
        # softmax saving the logsumexp, backward rebuilding y from x and lse
        self.call(ops["softmax_fwd_lse"])
        self.call(ops["softmax_bwd_lse"])
        torch.cuda.synchronize()
        ref = torch.logsumexp(f(x), 1)
        out["softmax_lse_L"] = worst((t["mlse"] - ref).abs(), 1e-5 * ref.abs() + 1e-5)
        out["softmax_lse_y_row_sums"] = float((f(t["my"]).sum(1) - 1).abs().max()) / 1e-2
        yr = torch.exp(xs - t["mlse"][rows, None])
        ref = yr * (gs - (gs * yr).sum(1, keepdim=True))
        sabs = (gs.abs() * yr).sum(1, keepdim=True)
        out["softmax_lse_dx_rows"] = worst((f(t["mdx"][rows]) - ref).abs(),
                                           2 ** -7 * ref.abs() + 1e-4 * yr * (gs.abs() + sabs) + 1e-30)
        # split cross-entropy: statistics forward, backward from the saved lse (dloss = 1)
        self.call(ops["softmax_xent_fwd"])
        self.call(ops["softmax_xent_bwd"])
        torch.cuda.synchronize()
        R = t["z"].shape[0]
        out.update(self._check_xent(t["loss"], t["rlse"], t["dz2"], float(t["dloss"].item()) / R,
                                    tag="softmax_xent_split"))
        # LayerNorm and RMSNorm: sampled rows of y, the statistics, and dw (db)
        w, b = f(t["nw"]), f(t["nb"])
        for name, rms in (("layernorm", False), ("rmsnorm", True)):
            self.call(ops[name + "_fwd"])
            self.call(ops[name + "_bwd"])
            torch.cuda.synchronize()
            eps = 1e-6 if rms else 1e-5
            X = f(x)
            if rms:
                rstd = torch.rsqrt((X * X).mean(1) + eps)
                xhat = X * rstd[:, None]
                ref_y = xhat[rows] * w
            else:
                mu = X.mean(1)
                rstd = torch.rsqrt(((X - mu[:, None]) ** 2).mean(1) + eps)
                xhat = (X - mu[:, None]) * rstd[:, None]
                ref_y = xhat[rows] * w + b
                out["layernorm_mean"] = worst((t["nmean"] - mu).abs(), 1e-5 * X.abs().mean(1) + 1e-30)
            out[f"{name}_rstd"] = worst((t["nrstd"] - rstd).abs(), 1e-4 * rstd)
            out[f"{name}_y_rows"] = worst((f(t["my"][rows]) - ref_y).abs(),
                                          2 ** -7 * ref_y.abs() + 1e-4 * (xhat[rows] * w).abs() + 1e-30)
            G = f(dy)
            out[f"{name}_dw"] = worst((t["ndw"] - (G * xhat).sum(0)).abs(), 1e-4 * (G * xhat).abs().sum(0) + 1e-30)
            if not rms:
                out["layernorm_db"] = worst((t["ndb"] - G.sum(0)).abs(), 1e-4 * G.abs().sum(0) + 1e-30)
            del X, xhat, G
        # row gather (a bit copy) and its scatter-add
        self.call(ops["gather_rows_fwd"])
        self.call(ops["gather_rows_bwd"])
        torch.cuda.synchronize()
        idx = t["e_idx"].long()
        out["gather_rows_y_exact"] = 0.0 if torch.equal(t["e_y"], t["e_tab"][idx]) else float("inf")
        G = f(t["e_dy"])
        ref = G.sum(0)
        out["gather_rows_dtable_column_sums"] = worst((t["e_dt"].sum(0) - ref).abs(), 1e-4 * G.abs().sum(0) + 1e-30)
        unsel = torch.bincount(idx, minlength=t["e_dt"].shape[0]) == 0
        out["gather_rows_dtable_zero_rows"] = 0.0 if not bool(t["e_dt"][unsel].any()) else float("inf")
        out["gather_rows_n_invalid"] = 0.0 if int(t["e_ninv"].item()) == 0 else float("inf")
        return out


def protocol_items(wb):
    """(label, bytes, elements, launch) in launch order: every op of the step and
    of the extras, the copy of the largest op's bytes at every shape of the
    sweep, and a copy of each op's own byte count at vjp_copy's shape."""
    items = [(o[0], o[3], o[4], (lambda o=o: wb.call(o))) for o in wb.ops + wb.extra_ops]
    big = 2 * wb.copy_half
    for vpl, wg in COPY_SHAPES:
        items.append((f"copy_sweep {vpl}x{wg}", big, big, lambda v=vpl, g=wg: wb.copy(big // 2, v, g)))
    for o in wb.ops + wb.extra_ops:
        nb = min(o[3] // 32 * 16, wb.copy_half)
        items.append((f"copy_matched {o[0]}", 2 * nb, 2 * nb, lambda n=nb: wb.copy(n)))
    return items


def run_protocol(wb, items, log_every=10):
    """Each item PROTOCOL_WARM + PROTOCOL_REPS times: 1 GiB of plain stores
    (torch's fill, one kernel) that evict L2 and the 256 MB Infinity Cache,
    then the item's launches, then a device synchronisation.  HIP events on the
    launch stream bracket the item's launches; returns their times (ms)."""
    torch = wb.torch
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=wb.ca.device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for k, (label, _, _, launch) in enumerate(items):
        ts = []
        for r in range(PROTOCOL_WARM + PROTOCOL_REPS):
            flush.fill_(r % 251)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            if r >= PROTOCOL_WARM:
                ts.append(e0.elapsed_time(e1))
        out.append(ts)
        if k % log_every == 0:
            print(f"[bench protocol] {k + 1}/{len(items)} {label}", file=sys.stderr, flush=True)
    del flush
    return out


def _median(v):
    v = sorted(v)
    n = len(v)
    return 0.5 * (v[(n - 1) // 2] + v[n // 2]) if n else float("nan")


def protocol_child(plan_file) -> int:
    """Runs the protocol (under rocprofv3, started by the parent): one marker
    copy of 4 KiB through unaligned pointers (the only byte-loop copy_bytes
    launch), then every item; writes the item labels and the event medians to
    plan_file."""
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wb = Workbench(dev)
    items = protocol_items(wb)
    for it in items:                       # one untimed pass of everything
        it[3]()
    torch.cuda.synchronize()
    wb.copy(4096, offset=1)                # marker (byte-loop copy kernel): the protocol starts after it
    torch.cuda.synchronize()
    times = run_protocol(wb, items)
    with open(plan_file, "w") as f:
        json.dump({"labels": [it[0] for it in items],
                   "event_median_ms": [_median(t) for t in times]}, f)
    return 0


def parse_protocol_trace(csv_path, labels):
    """Kernel durations of the protocol from a rocprofv3 kernel trace: after
    the marker copy (the copy_bytes launch), every fill kernel (the
    flush) opens a launch group; groups follow the labels in order, each
    PROTOCOL_WARM + PROTOCOL_REPS times.  Returns, per label, the median over
    the timed groups of the summed kernel durations (ms) and the median of
    each kernel's duration."""
    import csv

    with open(csv_path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    start = next(i for i, r in enumerate(rows) if "copy_bytes" in r["Kernel_Name"])
    groups = []
    for r in rows[start + 1:]:
        name = r["Kernel_Name"]
        if "FillFunctor" in name:
            groups.append([])
        elif groups:
            groups[-1].append((name, (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6))
    per = PROTOCOL_WARM + PROTOCOL_REPS
    if len(groups) != per * len(labels):
        raise RuntimeError(f"trace has {len(groups)} launch groups, expected {per * len(labels)}")
    out = {}
    for k, label in enumerate(labels):
        gs = groups[k * per + PROTOCOL_WARM:(k + 1) * per]
        kern = {}
        for g in gs:
            for name, ms in g:
                kern.setdefault(name, []).append(ms)
        out[label] = {"ms": _median([sum(ms for _, ms in g) for g in gs]),
                      "kernels": {n: {"median_ms": round(_median(v), 5), "launches": len(v)}
                                  for n, v in kern.items()}}
    return out


def under_profiler() -> bool:
    return any(k.startswith("ROCPROF") for k in os.environ)


def protocol_via_rocprof(timeout=300):
    """The protocol in a child process under rocprofv3 --kernel-trace, started
    before this process uses the GPU.  Returns (per-label results, command) or
    (None, reason)."""
    import glob
    import shutil
    import subprocess
    import tempfile

    exe = shutil.which("rocprofv3")
    if exe is None:
        return None, "rocprofv3 not found"
    tmp = tempfile.mkdtemp(prefix="vjp_protocol_")
    plan = os.path.join(tmp, "plan.json")
    cmd = [exe, "--kernel-trace", "--output-format", "csv", "-d", tmp, "-o", "protocol", "--",
           sys.executable, os.path.abspath(__file__), "--protocol-child", plan]
    try:
        r = subprocess.run(cmd, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE, text=True,
                           timeout=timeout)
        if not os.path.exists(plan):
            tail = (r.stderr or "")[-600:]
            return None, f"protocol child exited {r.returncode} without results: {tail}"
        with open(plan) as f:
            labels = json.load(f)["labels"]
        csvs = glob.glob(os.path.join(tmp, "**", "protocol_kernel_trace.csv"), recursive=True)
        if not csvs:
            return None, "no kernel trace written"
        return parse_protocol_trace(csvs[0], labels), " ".join(
            ["rocprofv3", "--kernel-trace", "--output-format", "csv", "-d", "<tmp>", "-o", "protocol",
             "--", "python3", "bench.py", "--protocol-child", "<tmp>/plan.json"])
    except Exception as exc:  # the event protocol in this process replaces it
        return None, f"{type(exc).__name__}: {exc}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def op_row(name, ms, nbytes, nelem, **extra):
    gbs = nbytes / (ms * 1e-3) / 1e9
    row = {"op": name, "ms": round(ms, 5), "bytes": nbytes, "GB/s": round(gbs, 1),
           "frac_of_peak": round(gbs / PEAK_GBS, 4), "elements_per_s": round(nelem / (ms * 1e-3), 1)}
    row.update(extra)
    return row


def pair_rows(pairs, by_name, copy_gbs, matched_ms=None):
    out = []
    for pname, members in pairs:
        if not all(m in by_name for m in members):
            continue
        ms = sum(by_name[m]["ms"] for m in members)
        nbytes = sum(by_name[m]["bytes"] for m in members)
        row = op_row(pname, ms, nbytes, sum(by_name[m]["elements_per_s"] * by_name[m]["ms"] * 1e-3
                                            for m in members))
        del row["elements_per_s"]
        row["frac_of_copy"] = round(row["GB/s"] / copy_gbs, 4) if copy_gbs else None
        if matched_ms is not None:
            mm = sum(matched_ms[m] for m in members)
            row["matched_copy_ms"] = round(mm, 5)
            row["frac_of_matched_copy"] = round(mm / ms, 4)
        out.append(row)
    return out


def protocol_summary_md(res, source, command, path):
    """Markdown table of the protocol's per-kernel medians (written for profiles/)."""
    lines = [f"# Fwd+bwd pairs, flushed: {source}", "",
             f"Command: `python3 bench.py --protocol-summary <out>/{os.path.basename(path)}` (its "
             "protocol child ran "
             f"`{command}`).", "",
             f"Each launch group ran {PROTOCOL_WARM} + {PROTOCOL_REPS} times after 1 GiB of plain "
             "stores (torch fill) that evict L2 and the Infinity Cache; medians over the last "
             f"{PROTOCOL_REPS}.", "",
             "| Group | Kernel | Launches | Median µs |", "|---|---|---|---|"]
    for label, r in res.items():
        for name, k in r["kernels"].items():
            lines.append(f"| {label} | `{name[:90]}` | {k['launches']} | {k['median_ms'] * 1e3:.2f} |")
        lines.append(f"| {label} | (sum) | | {r['ms'] * 1e3:.2f} |")
    return "\n".join(lines) + "\n"


COUNTER_CMD = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc_{c} -o run -- python3 bench.py "
               "--protocol off --steps 2 --warmup 1 --no-cpu-baseline --calib-copy")


def counters_summary(fetch_csv, write_csv, md_path, json_path):
    """HBM bytes per kernel from two rocprofv3 counter runs of this script
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the
    same counter reads for the 1 GiB device copy that --calib-copy runs
    (rocclr copyBuffer), against each kernel's algorithmic bytes.  Writes the
    markdown table and the roofline op's bytes per launch (with the digest of
    its sources) as JSON."""
    import csv
    import re

    def load(path, counter):
        d = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                n = r["Kernel_Name"].replace("void ", "").replace("(anonymous namespace)::", "")
                if "rocclr_copyBuffer" in n:
                    n = "copyBuffer"
                elif "vjp" in n:
                    n = re.sub(r"\(.*", "", n).replace("vjp::", "")
                    n = re.sub(r"^_ZN3vjp12_GLOBAL__N_1\d+", "", n)
                else:
                    continue
                d.setdefault((n, int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in d.items()}

    f, w = load(fetch_csv, "FETCH_SIZE"), load(write_csv, "WRITE_SIZE")
    calib = max((k for k in f if k[0] == "copyBuffer"), key=lambda k: f[k])
    ff, fw = f[calib] / (1 << 20), w[calib] / (1 << 20)
    RX, CX, RM, CM, NW, DW = 16384, 32000, 32768, 4096, 1048576, 256
    algo = {
        "xent_resident<bf16, 8, 16, 4, false, true>": 2 * RX * CX * 2 + RX * 4 + RX * 12,
        "xent_resident<bf16, 8, 8, 8, false, false>": RX * CX * 2 + RX * 4 + RX * 8,
        "xent_bwd_kernel<bf16, 8, 4, 1024>": 2 * RX * CX * 2 + RX * 8 + 4,
        "xent_finalize_kernel": RX * 8 + 8,
        "ws_bwd_kernel<bf16, 8, 4>": NW * 2 + 2 * NW * DW * 2 + DW * 2 + 1024 * DW * 4,
        "ws_fwd_kernel<bf16, 8, 4, false>": NW * DW * 2 + DW * 2 + NW * 2,
        "softmax_bwd_resident<bf16, 8, 8, 1, false>": 3 * RM * CM * 2,
        "softmax_bwd_resident<bf16, 8, 4, 2, true>": 3 * RM * CM * 2 + RM * 4,
        "softmax_fwd_resident<bf16, 8, 4, 2, true>": 2 * RM * CM * 2,
        "norm_fwd_resident<bf16, 8, 4, 2, false, 2, 2>": 2 * RM * CM * 2 + 2 * CM * 2 + RM * 8,
        "norm_fwd_resident<bf16, 8, 4, 2, true, 1, 2>": 2 * RM * CM * 2 + CM * 2 + RM * 4,
        "norm_bwd_tile<bf16, 8, 8, 1, false>": 3 * RM * CM * 2 + CM * 2 + RM * 8 + 512 * 2 * CM * 4,
        "norm_bwd_tile<bf16, 8, 8, 1, true>": 3 * RM * CM * 2 + CM * 2 + RM * 4 + 512 * CM * 4,
        "silu_fwd_kernelIDF16_Li8ELi8EEEvPKT_PKfPS2_ll": 2 * (1 << 24) * 2 + 4,
        "silu_bwd_kernelIDF16_Li8ELi2EEEvPKT_S4_PKfPS2_Pfll": 3 * (1 << 24) * 2 + 4 + 4096 * 4,
        "reduce_scalar_kernel": 4096 * 4 + 4,
        "gather_rows_fwd<bf16, 8>": 2 * 16384 * 4096 * 2 + 16384 * 4,
        "copy_vec16<4>": None,
    }
    algo_grid = {  # the stage-2 reduction, by its grid (columns / 32 workgroups of 1024 threads)
        ("reduce_partials_kernel<true>", 8 * 1024): 1024 * DW * 4 + DW * 4,
        ("reduce_partials_kernel<true>", 256 * 1024): 512 * 2 * CM * 4 + 2 * CM * 4,
        ("reduce_partials_kernel<true>", 128 * 1024): 512 * CM * 4 + CM * 4,
    }
    cmd_f, cmd_w = COUNTER_CMD.format(c="FETCH_SIZE"), COUNTER_CMD.format(c="WRITE_SIZE")
    lines = ["# HBM traffic counters per kernel", "",
             "Commands (one counter per run; `--calib-copy` runs a 1 GiB device copy for the "
             "calibration):", "", f"`{cmd_f}`", "", f"`{cmd_w}`", "",
             f"Summarised by `python3 bench.py --counters-summary <FETCH_SIZE csv> <WRITE_SIZE csv> "
             f"{md_path} {json_path}`.", "",
             f"Calibration: the 1 GiB copy reads FETCH_SIZE {f[calib]:.1f} KiB (factor {ff:.4f} of "
             f"the bytes read) and WRITE_SIZE {w[calib]:.1f} KiB (factor {fw:.4f} of the bytes "
             "written); every kernel's counters are divided by these factors.", "",
             f"Cross-entropy source digest: {source_digest()}", "",
             "| kernel | grid (threads) | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes (scaled) | "
             "written bytes (scaled) | algorithmic bytes | traffic / algorithmic |",
             "|---|---|---|---|---|---|---|---|"]
    for k in sorted(f, key=lambda k: -f[k]):
        if k[0] == "copyBuffer":
            continue
        rd, wr = f[k] / ff * 1024, w.get(k, 0.0) / fw * 1024
        a = algo_grid.get(k) or algo.get(k[0])
        if k[0].startswith("copy_vec16"):
            a = round(rd + wr)      # a copy: bytes read = bytes written
        ratio = f"{(rd + wr) / a:.4f}" if a else "-"
        lines.append(f"| {k[0]} | {k[1]} | {f[k]:.1f} | {w.get(k, 0.0):.1f} | {rd:.4g} | {wr:.4g} | "
                     f"{a if a else '-'} | {ratio} |")
    lines += ["", "The row gather reads less than its algorithmic bytes: its 16384 Zipf-distributed ids "
              "repeat table rows, and repeated rows are served from L2.  The scatter-add's dy reads are "
              "split between chunk_sums (positions in runs longer than 32) and scatter_listed_rows (the "
              "rest); its writes, the whole fp32 table of 32000 x 4096 x 4 bytes, are split between the "
              "zero rows written beside the plan (radix_pass_fused, plan_tail) and scatter_listed_rows "
              "(the rest of the zero rows and the selected rows)."]
    with open(md_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    main_k = next(k for k in f if k[0] == "xent_resident<bf16, 8, 16, 4, false, true>")
    fin_k = next(k for k in f if k[0] == "xent_finalize_kernel")
    tb = (f[main_k] / ff + w[main_k] / fw + f[fin_k] / ff + w[fin_k] / fw) * 1024
    with open(json_path, "w") as fh:
        json.dump({"op": "softmax_xent_fwd_bwd", "kernels": [main_k[0], fin_k[0]],
                   "source_digest": source_digest(), "fetch_kib": f[main_k] + f[fin_k],
                   "write_kib": w[main_k] + w[fin_k], "fetch_factor": ff, "write_factor": fw,
                   "bytes_per_launch": round(tb),
                   "algorithmic_bytes": algo[main_k[0]] + algo[fin_k[0]],
                   "commands": [cmd_f, cmd_w]}, fh, indent=1)
    return 0


STATS_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/prof -o run -- "
             "python3 bench.py --protocol off --no-cpu-baseline --steps 10 --warmup 3")


def stats_summary(stats_csv, bench_json, md_path):
    """Markdown table of a rocprofv3 --stats kernel summary of the warm step
    (STATS_CMD), with the bench line that run printed: the roofline kernel's
    average duration there is the one its live HIP events are checked against."""
    import csv

    with open(stats_csv) as f:
        rows = list(csv.DictReader(f))
    with open(bench_json) as f:
        line = json.loads([ln for ln in f if ln.startswith("{")][-1])
    rf = line["roofline"]
    ev_us = rf["bytes"] / (rf["achieved"] * 1e9) * 1e6 if "bytes" in rf else None
    lines = ["# Warm step: rocprofv3 kernel statistics", "",
             f"Command: `{STATS_CMD}` (kernel durations over the warmup, the per-op pass, the timed "
             "steps, the widened rows and the warm copies; no flushed protocol).", "",
             f"Summarised by `python3 bench.py --stats-summary <kernel_stats.csv> <bench line> {md_path}`.",
             "", f"That run's bench line: {line['ms_per_step']} ms per step, roofline op "
             f"{rf['kernel']} at {rf['achieved']} GB/s from HIP events around its launches in the "
             f"timed steps ({rf['frac']} of 8 TB/s)."]
    if ev_us is not None:
        lines.append(f"The events give {ev_us:.1f} µs per launch of that op.")
    lines += ["", "| Kernel | Calls | Average µs | Min µs | Max µs | Share of GPU time |",
              "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f}% |")
    with open(md_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-scale", type=float, default=1.0)
    ap.add_argument("--protocol", choices=["rocprof", "events", "off"], default="rocprof",
                    help="flushed per-op medians: kernel durations from a rocprofv3 child "
                         "(default; HIP events in this process when the child fails or this "
                         "process already runs under a profiler), HIP events only, or none")
    ap.add_argument("--protocol-summary", metavar="PATH",
                    help="also write the per-kernel medians of the protocol as markdown")
    ap.add_argument("--protocol-child", metavar="PLAN", help=argparse.SUPPRESS)
    ap.add_argument("--counters-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "MD", "JSON"),
                    help="summarise two rocprofv3 counter runs of this script (no GPU used)")
    ap.add_argument("--stats-summary", nargs=3, metavar=("STATS_CSV", "BENCH_JSON", "MD"),
                    help="summarise a rocprofv3 --stats run of this script (no GPU used)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy before timing (counter calibration)")
    args = ap.parse_args()
    if args.protocol_child:
        return protocol_child(args.protocol_child)
    if args.counters_summary:
        return counters_summary(*args.counters_summary)
    if args.stats_summary:
        return stats_summary(*args.stats_summary)
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the ops shard by rows with no exchange except one small grad_w all-reduce, "
              "which is not built here)", file=sys.stderr)
        return 2

    # The flushed protocol first, in a child under rocprofv3, before this
    # process touches the GPU.
    proto, proto_source, proto_note = None, None, None
    if args.protocol == "rocprof" and not under_profiler():
        print("[bench] protocol child under rocprofv3 (flushed per-op medians)", file=sys.stderr,
              flush=True)
        proto, proto_note = protocol_via_rocprof()
        if proto is not None:
            proto_source = "rocprofv3 kernel trace (sum of the kernel durations of each launch group)"
        else:
            print(f"[bench] rocprofv3 protocol unavailable: {proto_note}", file=sys.stderr, flush=True)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] device {torch.cuda.get_device_name(dev)}; generating inputs", file=sys.stderr, flush=True)
    wb = Workbench(dev)
    ops = wb.ops
    step_bytes = sum(o[3] for o in ops)

    def step(evs=None):
        for i, op in enumerate(ops):
            if evs is not None:
                evs[i][0].record()
            wb.call(op)
            if evs is not None:
                evs[i][1].record()

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # Per-op breakdown of the warm step: a separate pass with HIP events around
    # every op (the records between the kernels slow the step by ~7%, so this
    # pass is not the timed one); it also picks the op with the largest share
    # of the step (the roofline kernel).
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    per_op = [op_row(o[0], sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps))
                     / args.steps, o[3], o[4]) for i, o in enumerate(ops)]
    i_dom = max(range(len(ops)), key=lambda i: per_op[i]["ms"])
    print(f"[bench] per-op pass done; timing {args.steps} steps", file=sys.stderr, flush=True)

    # The timed region: K steps with HIP events around the roofline kernel only
    # (on its launch stream), bracketed by device synchronisations.
    dev_evs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for i, op in enumerate(ops):
            if i == i_dom:
                dev_evs[k][0].record()
            wb.call(op)
            if i == i_dom:
                dev_evs[k][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / args.steps * 1e3
    ms_dom = sum(ev[0].elapsed_time(ev[1]) for ev in dev_evs) / args.steps
    dom = op_row(ops[i_dom][0], ms_dom, ops[i_dom][3], ops[i_dom][4])
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step; {dom['op']} {ms_dom * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    checks = wb.check_step()

    # Widened rows (warm, events around each op), after and outside the step.
    n_extra = max(3, args.steps // 2)
    xevs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
             for _ in wb.extra_ops] for _ in range(n_extra + 1)]
    for k in range(n_extra + 1):          # the first round is a warmup
        for i, op in enumerate(wb.extra_ops):
            xevs[k][i][0].record()
            wb.call(op)
            xevs[k][i][1].record()
    torch.cuda.synchronize()
    extras = [op_row(o[0], sum(xevs[k][i][0].elapsed_time(xevs[k][i][1]) for k in range(1, n_extra + 1))
                     / n_extra, o[3], o[4]) for i, o in enumerate(wb.extra_ops)]
    print(f"[bench] timed the widened rows ({n_extra} rounds)", file=sys.stderr, flush=True)
    checks.update(wb.check_extras())
    bad = {k: v for k, v in checks.items() if not v <= 1.0}
    if bad:
        print(f"[bench] output checks failed (error / bound): {bad}", file=sys.stderr, flush=True)
        return 1
    print(f"[bench] {len(checks)} output checks passed (worst error / bound "
          f"{max(checks.values()):.3f})", file=sys.stderr, flush=True)

    # Flushed protocol: from the rocprofv3 child, else HIP events here.
    items = protocol_items(wb)
    if proto is None and args.protocol != "off":
        times = run_protocol(wb, items)
        proto = {it[0]: {"ms": _median(t)} for it, t in zip(items, times)}
        proto_source = "HIP events on the launch stream around each launch group"
        if proto_note is None and under_profiler():
            proto_note = "this process runs under a profiler"
    result_protocol, pairs_cold, extra_pairs_cold, copy_ceiling = None, None, None, None
    if proto is not None:
        by_label = {it[0]: it for it in items}
        per_op_cold = [op_row(o[0], proto[o[0]]["ms"], o[3], o[4]) for o in ops]
        extras_cold = [op_row(o[0], proto[o[0]]["ms"], o[3], o[4]) for o in wb.extra_ops]
        sweep = []
        for vpl, wg in COPY_SHAPES:
            lab = f"copy_sweep {vpl}x{wg}"
            sweep.append({"vectors_per_lane": vpl, "max_workgroups": wg, "ms": round(proto[lab]["ms"], 5),
                          "GB/s": round(by_label[lab][1] / (proto[lab]["ms"] * 1e-3) / 1e9, 1)})
        best = max(sweep, key=lambda c: c["GB/s"])
        copy_gbs = best["GB/s"]
        matched = {o[0]: proto[f"copy_matched {o[0]}"]["ms"] for o in ops + wb.extra_ops}
        by_name = {r["op"]: r for r in per_op_cold + extras_cold}
        pairs_cold = pair_rows(PAIRS, by_name, copy_gbs, matched)
        extra_pairs_cold = pair_rows(EXTRA_PAIRS, by_name, copy_gbs, matched)
        copy_ceiling = {"GB/s": copy_gbs, "bytes": 2 * wb.copy_half,
                        "best_shape": {"vectors_per_lane": best["vectors_per_lane"],
                                       "max_workgroups": best["max_workgroups"]},
                        "sweep": sweep,
                        "kernel": "vjp_copy_shaped (16-byte nontemporal loads and stores), flushed, median"}
        result_protocol = {"source": proto_source, "note": proto_note, "reps": PROTOCOL_REPS,
                           "warmup_reps": PROTOCOL_WARM, "statistic": "median",
                           "flush": "1 GiB of plain stores (torch fill) before every launch group",
                           "per_op": per_op_cold, "extras": extras_cold}
        if args.protocol_summary and "kernels" in next(iter(proto.values())):
            with open(args.protocol_summary, "w") as f:
                f.write(protocol_summary_md(proto, proto_source, proto_note, args.protocol_summary))
        dom_cold = by_name[dom["op"]]
        print(f"[bench] protocol ({proto_source.split(' (')[0]}): "
              + ", ".join(f"{p['op']} {p['frac_of_peak']:.3f}" for p in pairs_cold),
              file=sys.stderr, flush=True)
    else:
        dom_cold = None

    # warm pairs, against the warm copy of the roofline op's bytes
    cevs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(6)]
    for ev in cevs:                       # the first copy is a warmup
        ev[0].record()
        wb.copy(wb.copy_half)
        ev[1].record()
    torch.cuda.synchronize()
    ms_copy = sum(ev[0].elapsed_time(ev[1]) for ev in cevs[1:]) / (len(cevs) - 1)
    warm_copy_gbs = 2 * wb.copy_half / (ms_copy * 1e-3) / 1e9
    pairs = pair_rows(PAIRS, {r["op"]: r for r in per_op}, warm_copy_gbs)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("op") == dom["op"] and tr.get("source_digest") == source_digest():
            traffic = tr.get("bytes_per_launch")
    value = step_bytes / (ms_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": ("bf16 (weighted_sum, softmax, softmax_xent), fp16 (scaled_silu); fp32 "
                          "parameter gradients, row statistics and partials; all arithmetic fp32"),
        "data": "synthetic (seeded normal draws on the device; uniform int32 targets)",
        "config": {
            "workload": ("one fwd+bwd of each op: weighted_sum bf16 1048576x256, scaled_silu "
                         "fp16 n=16777216, softmax bf16 32768x4096, softmax_xent bf16 16384x32000"),
            "step_bytes": step_bytes,
            "frac_of_peak": round(value / PEAK_GBS, 4),
        },
        "pairs_cold": pairs_cold,
        "extra_pairs_cold": extra_pairs_cold,
        "protocol": result_protocol,
        "copy_ceiling": copy_ceiling,
        "per_op": per_op,
        "pairs": pairs,
        "per_op_timing": "warm step: separate pass, HIP events around every op (not the timed steps)",
        "extras": extras,
        "roofline": {
            "kernel": dom["op"],
            "bound": "hbm",
            "achieved": dom["GB/s"],
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom["GB/s"] / PEAK_GBS, 4),
            "bytes": dom["bytes"],
            "us_per_launch": round(ms_dom * 1e3, 2),
            "traffic": traffic,
            "timing": "HIP events around the kernel's launches in the timed steps, mean",
            "frac_flushed_median": dom_cold["frac_of_peak"] if dom_cold else None,
            "frac_of_warm_copy": round(dom["GB/s"] / warm_copy_gbs, 4),
        },
        "cpu_baseline": None,
        "checks": {k: round(v, 4) for k, v in checks.items()},
    }
    del wb
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample (all cores, then one)", file=sys.stderr, flush=True)
        try:
            result["cpu_baseline"] = cpu_baseline(args.cpu_scale)
        except Exception as exc:
            result["cpu_baseline"] = {"error": f"{type(exc).__name__}: {exc}"}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
