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
read and write once; listed per op in `per_op`) divided by the measured step
time over K steps whose only instrumentation is one pair of HIP events
around the `roofline` op (the op with the largest share of the step), on the
stream the kernels are launched on; its `achieved` comes from those events.
The per-op breakdown (`per_op`) comes from a separate pass with events around
every op (those records slow each op slightly); `pairs` sums it per forward +
backward pair.  `per_op_cold` / `pairs_cold` time each op alone after 1 GiB
of writes that evict L2 and the 256 MB Infinity Cache (no op finds its
inputs, or an earlier op's pending write-back, in a cache).  `copy_ceiling` times the library's streaming copy
(vjp_copy) of as many bytes as the roofline op moves, half read and half
written, in the same process: the rate at which this GPU reads and writes
each byte once, which no kernel that moves its bytes once can beat by much;
`frac_of_copy` compares against it; `frac_of_matched_copy` compares each
pair with copies of each of its ops' own byte counts, one launch per op.  `cpu_baseline` times the fp64 CPU oracle on a
bounded sample of the same workloads on one host core.  `extras` times the
save-the-statistics variants (softmax forward writing the row logsumexp and
the backward rebuilding y from it; the split cross-entropy forward and
backward), LayerNorm / RMSNorm forward and backward on the softmax
workload's [32768, 4096] bf16 inputs, and the embedding gather with its
deterministic scatter-add backward (16384 Zipf token ids, 32000 x 4096
table), after and outside the step.

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
# share of the step) and the build flags: stored counter readings for it expire
# when any of them changes.
XENT_SOURCES = ("softmax_xent.hip", "reduce.hip", "rowops.hpp", "common.hpp")


def source_digest(files=XENT_SOURCES) -> str:
    """Hash of the named kernel sources and of the build script."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "row_wise_backward_amd", "csrc")
    paths = [os.path.join(csrc, f) for f in files]
    paths.append(os.path.join(ROOT, "row_wise_backward_amd", "build.py"))
    for path in paths:
        with open(path, "rb") as fh:
            h.update(os.path.basename(path).encode() + fh.read())
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

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-scale", type=float, default=1.0)
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy before timing (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(the ops shard by rows with no exchange except one small grad_w all-reduce, "
              "which is not built here)", file=sys.stderr)
        return 2

    import torch

    import row_wise_backward_amd as rwb
    import synth
    from synth.workloads import SILU_16M, SOFTMAX, WS_LARGE, XENT

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = rwb.lib
    print(f"[bench] device {torch.cuda.get_device_name(dev)}; generating inputs", file=sys.stderr, flush=True)

    # inputs (seeded, drawn on the device) and outputs
    n_ws, d_ws = WS_LARGE.shape
    wx = synth.normal_device((n_ws, d_ws), WS_LARGE.sigma_x, "bf16", WS_LARGE.seed, 0, dev)
    ww = synth.normal_device((d_ws,), WS_LARGE.sigma_w, "bf16", WS_LARGE.seed, 1, dev)
    wg = synth.normal_device((n_ws,), WS_LARGE.sigma_dy, "bf16", WS_LARGE.seed, 2, dev)
    wy = torch.empty(n_ws, dtype=torch.bfloat16, device=dev)
    wdx = torch.empty_like(wx)
    wdw = torch.empty(d_ws, dtype=torch.float32, device=dev)
    T_ws = rwb.vjp_weighted_sum_bwd_workspace_size(n_ws, d_ws) // (4 * d_ws)
    wws = torch.empty(rwb.vjp_weighted_sum_bwd_workspace_size(n_ws, d_ws), dtype=torch.uint8, device=dev)

    n_s = SILU_16M.shape[0]
    sx = synth.normal_device((n_s,), SILU_16M.sigma_x, "f16", SILU_16M.seed, 0, dev)
    sg = synth.normal_device((n_s,), SILU_16M.sigma_dy, "f16", SILU_16M.seed, 2, dev)
    sw = torch.tensor([SILU_16M.w_value], dtype=torch.float32, device=dev)
    sy, sdx = torch.empty_like(sx), torch.empty_like(sx)
    sdw = torch.empty(1, dtype=torch.float32, device=dev)
    T_s = rwb.vjp_scaled_silu_bwd_workspace_size(n_s) // 4
    sws = torch.empty(rwb.vjp_scaled_silu_bwd_workspace_size(n_s), dtype=torch.uint8, device=dev)

    r_m, c_m = SOFTMAX.shape
    mx = synth.normal_device((r_m, c_m), SOFTMAX.sigma_x, "bf16", SOFTMAX.seed, 0, dev)
    mg = synth.normal_device((r_m, c_m), SOFTMAX.sigma_dy, "bf16", SOFTMAX.seed, 2, dev)
    my, mdx = torch.empty_like(mx), torch.empty_like(mx)

    r_x, c_x = XENT.shape
    z = synth.normal_device((r_x, c_x), XENT.sigma_x, "bf16", XENT.seed, 0, dev)
    tg = synth.targets_device(r_x, c_x, XENT.seed, dev)
    dz = torch.empty_like(z)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    rmax = torch.empty(r_x, dtype=torch.float32, device=dev)
    rlse = torch.empty(r_x, dtype=torch.float32, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    xws = torch.empty(rwb.vjp_softmax_xent_workspace_size(r_x), dtype=torch.uint8, device=dev)
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
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    BF16, F16 = rwb.VJP_BF16, rwb.VJP_F16
    ops = [
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
    step_bytes = sum(o[3] for o in ops)

    def step(evs=None):
        for i, (name, fn, a, _, _) in enumerate(ops):
            if evs is not None:
                evs[i][0].record()
            st = fn(*a)
            if st != 0:
                raise RuntimeError(f"{name}: status {st} ({rwb.vjp_last_error()})")
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

    # Per-op breakdown: a separate pass with HIP events around every op.  The
    # event records between the kernels slow the step by ~7% and each op a
    # little, so this pass is not the timed one; it also picks the op with the
    # largest share of the step (the roofline kernel).
    evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    per_op = []
    for i, (name, _, _, nbytes, nelem) in enumerate(ops):
        ms = sum(evs[k][i][0].elapsed_time(evs[k][i][1]) for k in range(args.steps)) / args.steps
        gbs = nbytes / (ms * 1e-3) / 1e9
        per_op.append({"op": name, "ms": round(ms, 5), "bytes": nbytes, "GB/s": round(gbs, 1),
                       "frac_of_peak": round(gbs / PEAK_GBS, 4),
                       "elements_per_s": round(nelem / (ms * 1e-3), 1)})
    i_dom = max(range(len(ops)), key=lambda i: per_op[i]["ms"])

    # Cold per-op pass: before every op, 1 GiB of writes evicts L2 and the
    # 256 MB Infinity Cache, so no op finds its inputs, or the write-back of
    # an earlier op's outputs, in a cache.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    n_cold = max(3, args.steps // 2)
    cold_evs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                 for _ in ops] for _ in range(n_cold)]
    for k in range(n_cold):
        for i, (name, fn, a, _, _) in enumerate(ops):
            flush.fill_(k % 251)
            cold_evs[k][i][0].record()
            st = fn(*a)
            if st != 0:
                raise RuntimeError(f"{name}: status {st} ({rwb.vjp_last_error()})")
            cold_evs[k][i][1].record()
    torch.cuda.synchronize()
    del flush
    per_op_cold = []
    for i, (name, _, _, nbytes, nelem) in enumerate(ops):
        ms = sum(cold_evs[k][i][0].elapsed_time(cold_evs[k][i][1]) for k in range(n_cold)) / n_cold
        gbs = nbytes / (ms * 1e-3) / 1e9
        per_op_cold.append({"op": name, "ms": round(ms, 5), "bytes": nbytes, "GB/s": round(gbs, 1),
                            "frac_of_peak": round(gbs / PEAK_GBS, 4),
                            "elements_per_s": round(nelem / (ms * 1e-3), 1)})
    print(f"[bench] per-op passes done; timing {args.steps} steps", file=sys.stderr, flush=True)

    # The timed region: K steps with HIP events around the roofline kernel only
    # (on its launch stream), bracketed by device synchronisations.
    dev_evs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        for i, (name, fn, a, _, _) in enumerate(ops):
            if i == i_dom:
                dev_evs[k][0].record()
            st = fn(*a)
            if st != 0:
                raise RuntimeError(f"{name}: status {st} ({rwb.vjp_last_error()})")
            if i == i_dom:
                dev_evs[k][1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed / args.steps * 1e3
    ms_dom = sum(e[0].elapsed_time(e[1]) for e in dev_evs) / args.steps
    dom = dict(per_op[i_dom])
    dom["GB/s"] = round(dom["bytes"] / (ms_dom * 1e-3) / 1e9, 1)
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step; {dom['op']} {ms_dom * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    # Save-the-statistics variants (softmax with saved logsumexp, split
    # cross-entropy), timed after the step on the same inputs; not part of it.
    mlse = torch.empty(r_m, dtype=torch.float32, device=dev)
    dz2 = torch.empty_like(z)
    dloss = torch.ones(1, dtype=torch.float32, device=dev)
    # LayerNorm / RMSNorm on the softmax workload's shape (x = mx, dy = mg)
    nw = synth.normal_device((c_m,), 0.1, "bf16", SOFTMAX.seed, 1, dev) + 1.0
    nb = synth.normal_device((c_m,), 0.1, "bf16", SOFTMAX.seed, 3, dev)
    nmean = torch.empty(r_m, dtype=torch.float32, device=dev)
    nrstd = torch.empty(r_m, dtype=torch.float32, device=dev)
    ndw = torch.empty(c_m, dtype=torch.float32, device=dev)
    ndb = torch.empty(c_m, dtype=torch.float32, device=dev)
    T_ln = rwb.vjp_layernorm_bwd_workspace_size(r_m, c_m) // (8 * c_m)
    lnws = torch.empty(rwb.vjp_layernorm_bwd_workspace_size(r_m, c_m), dtype=torch.uint8, device=dev)
    T_rms = rwb.vjp_rmsnorm_bwd_workspace_size(r_m, c_m) // (4 * c_m)
    rmsws = torch.empty(rwb.vjp_rmsnorm_bwd_workspace_size(r_m, c_m), dtype=torch.uint8, device=dev)
    F32 = ctypes.c_float
    # Embedding lookup and its scatter-add backward (Zipf token ids)
    from synth.workloads import EMBED
    e_M, e_D = EMBED.shape
    e_V = EMBED.extra["V"]
    e_idx = torch.from_numpy(synth.zipf_indices(e_M, e_V, EMBED.seed, EMBED.extra["zipf_a"])).to(dev)
    e_tab = synth.normal_device((e_V, e_D), 1.0, "bf16", EMBED.seed, 0, dev)
    e_y = torch.empty((e_M, e_D), dtype=torch.bfloat16, device=dev)
    e_dy = synth.normal_device((e_M, e_D), 1.0, "bf16", EMBED.seed, 2, dev)
    e_dt = torch.empty((e_V, e_D), dtype=torch.float32, device=dev)
    e_ninv = torch.empty(1, dtype=torch.int32, device=dev)
    e_ws = torch.empty(rwb.vjp_gather_rows_bwd_workspace_size(e_M, e_V, e_D), dtype=torch.uint8,
                       device=dev)
    extra_ops = [
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
         (P(mg), c_m, P(mx), c_m, P(nw), P(nmean), P(nrstd), P(mdx), c_m, P(ndw), P(ndb), 0, r_m, c_m,
          F32(1e-5), BF16, BF16, P(lnws), lnws.numel(), stream),
         bytes_layernorm_bwd(r_m, c_m, T_ln), r_m * c_m),
        ("rmsnorm_fwd", L.vjp_rmsnorm_fwd,
         (P(mx), c_m, P(nw), P(my), c_m, P(nrstd), r_m, c_m, F32(1e-6), BF16, BF16, stream),
         bytes_rmsnorm_fwd(r_m, c_m), r_m * c_m),
        ("gather_rows_fwd", L.vjp_gather_rows_fwd,
         (P(e_tab), e_D, e_V, e_D, P(e_idx), e_M, P(e_y), e_D, BF16, stream),
         bytes_gather_fwd(e_M, e_D), e_M * e_D),
        ("gather_rows_bwd", L.vjp_gather_rows_bwd,
         (P(e_dy), e_D, P(e_idx), e_M, e_V, e_D, P(e_dt), e_D, 0, P(e_ninv), BF16, P(e_ws),
          e_ws.numel(), stream),
         bytes_gather_bwd(e_M, e_V, e_D), e_M * e_D),
        ("rmsnorm_bwd", L.vjp_rmsnorm_bwd,
         (P(mg), c_m, P(mx), c_m, P(nw), P(nrstd), P(mdx), c_m, P(ndw), 0, r_m, c_m, F32(1e-6), BF16,
          BF16, P(rmsws), rmsws.numel(), stream),
         bytes_rmsnorm_bwd(r_m, c_m, T_rms), r_m * c_m),
    ]
    n_extra = max(3, args.steps // 2)
    xevs = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
             for _ in extra_ops] for _ in range(n_extra + 1)]
    for k in range(n_extra + 1):          # the first round is a warmup
        for i, (name, fn, a, _, _) in enumerate(extra_ops):
            xevs[k][i][0].record()
            st = fn(*a)
            if st != 0:
                raise RuntimeError(f"{name}: status {st} ({rwb.vjp_last_error()})")
            xevs[k][i][1].record()
    torch.cuda.synchronize()
    extras = []
    for i, (name, _, _, nbytes, nelem) in enumerate(extra_ops):
        ms = sum(xevs[k][i][0].elapsed_time(xevs[k][i][1]) for k in range(1, n_extra + 1)) / n_extra
        gbs = nbytes / (ms * 1e-3) / 1e9
        extras.append({"op": name, "ms": round(ms, 5), "bytes": nbytes, "GB/s": round(gbs, 1),
                       "frac_of_peak": round(gbs / PEAK_GBS, 4),
                       "elements_per_s": round(nelem / (ms * 1e-3), 1)})
    print(f"[bench] timed the statistics-saving variants ({n_extra} rounds)", file=sys.stderr, flush=True)

    # Copy ceiling: vjp_copy (16-byte nontemporal loads and stores) of as many
    # bytes as the roofline op moves, half read and half written, in this
    # process: the rate at which this GPU reads and writes each byte once.
    half = dom["bytes"] // 32 * 16
    ca = torch.empty(half, dtype=torch.uint8, device=dev)
    cb = torch.empty_like(ca)
    cevs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
            for _ in range(6)]
    for e in cevs:                        # the first copy is a warmup
        e[0].record()
        st = L.vjp_copy(P(ca), P(cb), half, stream)
        if st != 0:
            raise RuntimeError(f"vjp_copy: status {st} ({rwb.vjp_last_error()})")
        e[1].record()
    torch.cuda.synchronize()
    ms_copy = sum(e[0].elapsed_time(e[1]) for e in cevs[1:]) / (len(cevs) - 1)
    copy_gbs = 2 * half / (ms_copy * 1e-3) / 1e9

    # Size-matched copies: a copy of each op's own byte count (half read, half
    # written) in its own launch, so that a small op is compared with a copy
    # that pays the same launch and ramp costs.  Successive copies move
    # through the buffers, so a small copy does not find its source in a cache.
    copy_ms_cache = {}

    def copy_ms(nbytes):
        n = min(nbytes // 32 * 16, half)
        if n not in copy_ms_cache:
            evs = [[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
                   for _ in range(6)]
            for k, e in enumerate(evs):
                off = (k * n) % (half - n + 16) // 16 * 16
                e[0].record()
                st = L.vjp_copy(ctypes.c_void_p(ca.data_ptr() + off),
                               ctypes.c_void_p(cb.data_ptr() + off), n, stream)
                if st != 0:
                    raise RuntimeError(f"vjp_copy: status {st} ({rwb.vjp_last_error()})")
                e[1].record()
            torch.cuda.synchronize()
            copy_ms_cache[n] = sum(e[0].elapsed_time(e[1]) for e in evs[1:]) / (len(evs) - 1)
        return copy_ms_cache[n]

    # Forward + backward pairs (from the per-op passes).
    def pair_figures(rows):
        by_name = {o["op"]: o for o in rows}
        out = []
        for pname, members in PAIRS:
            ms = sum(by_name[m]["ms"] for m in members)
            nbytes = sum(by_name[m]["bytes"] for m in members)
            gbs = nbytes / (ms * 1e-3) / 1e9
            ms_matched = sum(copy_ms(by_name[m]["bytes"]) for m in members)
            out.append({"op": pname, "ms": round(ms, 5), "bytes": nbytes, "GB/s": round(gbs, 1),
                        "frac_of_peak": round(gbs / PEAK_GBS, 4),
                        "frac_of_copy": round(gbs / copy_gbs, 4),
                        "matched_copy_ms": round(ms_matched, 5),
                        "frac_of_matched_copy": round(ms_matched / ms, 4)})
        return out

    pairs = pair_figures(per_op)
    pairs_cold = pair_figures(per_op_cold)
    del ca, cb

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
        "data": "synthetic (seeded normal draws on the device; uniform int32 targets)",
        "config": {
            "workload": ("one fwd+bwd of each op: weighted_sum bf16 1048576x256, scaled_silu "
                         "fp16 n=16777216, softmax bf16 32768x4096, softmax_xent bf16 16384x32000"),
            "step_bytes": step_bytes,
            "frac_of_peak": round(value / PEAK_GBS, 4),
        },
        "per_op": per_op,
        "pairs": pairs,
        "per_op_timing": "separate pass, HIP events around every op (not the timed steps)",
        "per_op_cold": per_op_cold,
        "pairs_cold": pairs_cold,
        "per_op_cold_timing": "each op alone after 1 GiB of writes that evict L2 and the Infinity Cache",
        "extras": extras,
        "roofline": {
            "kernel": dom["op"],
            "bound": "hbm",
            "achieved": dom["GB/s"],
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom["GB/s"] / PEAK_GBS, 4),
            "traffic": traffic,
        },
        "copy_ceiling": {
            "GB/s": round(copy_gbs, 1),
            "bytes": 2 * half,
            "kernel": "vjp_copy (16-byte nontemporal loads and stores), same process",
            "roofline_frac_of_copy": round(dom["GB/s"] / copy_gbs, 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(args.cpu_scale)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
