"""Seeded random configurations of every op against the oracle.

Shapes, padded or unaligned leading dimensions, activation and parameter
dtypes, tile sizes, accumulation and invalid indices are drawn from one
seeded generator per case, so that combinations the per-op suites do not list
one by one are covered too (for instance an invalid target falling in the
padding of a row's last vector).  Every case runs through the per-op suite's
own comparison, with that suite's tolerances.
"""
import numpy as np
import pytest

import synth
import test_gpu_gather as tg
import test_gpu_norms as tn
import test_gpu_scaled_silu as tss
import test_gpu_softmax as ts
import test_gpu_softmax_lse as tsl
import test_gpu_softmax_xent as tx
import test_gpu_softmax_xent_split as txs
import test_gpu_weighted_sum as tw

pytestmark = pytest.mark.gpu
N_CASES = 96
ACTS = ["f32", "f16", "bf16"]


def _rng(op, case):
    return np.random.default_rng([7100, op, case])


def _cols(g, hi):
    """Half the cases narrow (1 .. 299), half wide (300 .. hi)."""
    return int(g.integers(1, 300)) if g.integers(0, 2) == 0 else int(g.integers(300, hi))


def _layout(g, cols):
    """(ld, offset): natural, rows padded by 1 .. 16 elements, or an
    unaligned base with rows padded by 0 .. 8 elements."""
    kind = int(g.integers(0, 3))
    if kind == 0:
        return None, 0
    if kind == 1:
        return cols + int(g.integers(1, 17)), 0
    return cols + int(g.integers(0, 9)), int(g.integers(1, 8))


def _targets(g, rows, C):
    """Uniform targets, about one row in four invalid: negative, C, inside the
    last vector's padding (C + 0 .. 7), or far out of range."""
    t = g.integers(0, C, size=rows).astype(np.int64)
    for r in range(rows):
        if g.integers(0, 4) == 0:
            t[r] = [-1, C, C + int(g.integers(0, 8)), 2 ** 31 - 1][int(g.integers(0, 4))]
    return t.astype(np.int32)


@pytest.mark.parametrize("case", range(N_CASES))
def test_softmax_random(gpu_lib, case):
    g = _rng(1, case)
    rows, cols, act = int(g.integers(1, 40)), _cols(g, 9000), ACTS[case % 3]
    ld, off = _layout(g, cols)
    ts.run_case(gpu_lib, rows, cols, act, seed=7100 + case, ld=ld, offset=off)
    tsl.run_case(gpu_lib, rows, cols, act, seed=7200 + case, ld=ld, offset=off)


@pytest.mark.parametrize("case", range(N_CASES))
def test_softmax_xent_random(gpu_lib, case):
    g = _rng(2, case)
    rows, C, act = int(g.integers(1, 24)), _cols(g, 40000), ACTS[case % 3]
    ld, off = _layout(g, C)
    t = _targets(g, rows, C)
    tx.run_case(gpu_lib, rows, C, act, seed=7300 + case, ld=ld, offset=off, targets=t)
    txs.run_case(gpu_lib, rows, C, act, seed=7400 + case, ld=ld, offset=off, targets=t,
                 dloss=float(g.choice([1.0, -0.5, 3.0])))


@pytest.mark.parametrize("case", range(N_CASES))
def test_norms_random(gpu_lib, case):
    g = _rng(3, case)
    rows, cols = int(g.integers(1, 40)), _cols(g, 9000)
    act, wdt = ACTS[case % 3], ACTS[int(g.integers(0, 3))]
    ld, off = _layout(g, cols)
    for kind in ("ln", "rms"):
        tn.run_case(gpu_lib, kind, rows, cols, act, wdt, seed=7500 + case, ld=ld, offset=off,
                    saved=bool(g.integers(0, 2)), accumulate=bool(g.integers(0, 2)),
                    param_offset=int(g.integers(0, 2)))


@pytest.mark.parametrize("case", range(N_CASES))
def test_weighted_sum_random(gpu_lib, case):
    g = _rng(4, case)
    n, d = int(g.integers(1, 3000)), _cols(g, 1200)
    act, wdt = ACTS[case % 3], ACTS[int(g.integers(0, 3))]
    ld, off = _layout(g, d)
    rpt = int(g.choice([0, 1, 7, 32, int(g.integers(1, 500))]))
    tw.run_case(gpu_lib, n, d, act, wdt, seed=7600 + case, ld=ld, offset=off, rows_per_tile=rpt,
                accumulate=bool(g.integers(0, 2)))


@pytest.mark.parametrize("case", range(N_CASES))
def test_scaled_silu_random(gpu_lib, case):
    g = _rng(5, case)
    n, act = int(g.integers(1, 200000)), ACTS[case % 3]
    x = synth.normal((n,), float(g.choice([0.5, 2.0, 8.0])), act, 7700 + case, synth.STREAM_X)
    dy = synth.normal((n,), 1.0, act, 7700 + case, synth.STREAM_DY)
    tss.check(gpu_lib, x, dy, float(g.choice([0.75, -1.5, 3.0])), act,
              accumulate=bool(g.integers(0, 2)), offset=int(g.integers(0, 8)))


@pytest.mark.parametrize("case", range(N_CASES))
def test_gather_random(gpu_lib, case):
    g = _rng(6, case)
    M = int(g.choice([int(g.integers(1, 3000)), int(g.integers(15000, 20000))]))
    # (the oracle's fp64 copy of dy stays below ~50 MB)
    V, act = int(g.integers(1, 5000)), ACTS[case % 3]
    D = _cols(g, 3000) if M < 3000 else int(g.integers(1, 300))
    ld, off = _layout(g, D)
    kind = ["zipf", "uniform", "one_row", "invalid_mix"][int(g.integers(0, 4))]
    tg.run_case(gpu_lib, M, V, D, act, seed=7800 + case, kind=kind, ld=ld, offset=off,
                accumulate=bool(g.integers(0, 2)))
