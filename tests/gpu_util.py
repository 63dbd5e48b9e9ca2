"""Helpers shared by the GPU parity tests: device transfer, padded layouts, guards.

Inputs always come from :mod:`synth` on the host and expected values from
:mod:`oracle`; the HIP path only produces the values under test.
"""
from __future__ import annotations

import numpy as np
import torch

import synth

DEV = "cuda:0"
GUARD = 4096  # elements of sentinel on each side of a guarded output


def to_dev(arr, dtype):
    return synth.to_torch(arr, dtype, DEV)


def to_host(t, dtype):
    torch.cuda.synchronize()
    return synth.from_torch(t, dtype)


# Every 2-D buffer made by padded() / empty_padded() sits between sentinel
# bands of GUARD elements (at least 4 KiB); the gaps between the rows of a
# padded layout hold the sentinel too.  Each one is registered here, and
# after every GPU test (conftest) all registered bands and gaps must still
# hold their sentinel: a write outside an output, or into a gap, fails.
_GUARDS = []


class Guard2D:
    """Sentinel bands before and after a [rows, cols] row-major view with row
    stride ld, and the sentinel-filled gaps between its rows."""

    def __init__(self, rows, cols, dtype, ld, offset, name):
        self.rows, self.cols, self.ld, self.name = rows, cols, ld, name
        tdt = synth.torch_dtype(dtype)
        self.s = Guarded.SENTINEL[tdt]
        self.base = GUARD + offset
        self.span = max(rows - 1, 0) * ld + cols if rows and cols else 0
        self.buf = torch.full((self.base + self.span + GUARD,), self.s, dtype=tdt, device=DEV)
        self.t = self.buf.as_strided((rows, cols), (ld, 1), self.base)
        _GUARDS.append(self)

    def intact(self) -> bool:
        torch.cuda.synchronize()
        ok = bool((self.buf[:self.base] == self.s).all().item())
        ok = ok and bool((self.buf[self.base + self.span:] == self.s).all().item())
        if ok and self.rows > 1 and self.ld > self.cols and self.cols > 0:
            gaps = self.buf.as_strided((self.rows - 1, self.ld - self.cols), (self.ld, 1),
                                       self.base + self.cols)
            ok = bool((gaps == self.s).all().item())
        return ok


def guards_broken():
    """Names of the registered buffers whose bands or row gaps changed; clears
    the registry."""
    bad = [g.name for g in _GUARDS if not g.intact()]
    _GUARDS.clear()
    return bad


def padded(arr2d, dtype, ld=None, offset=0):
    """Upload a [rows, cols] storage array into a device buffer with row stride
    ``ld`` (>= cols) starting ``offset`` elements past the leading sentinel
    band, so that leading dimensions and base alignments other than the
    natural ones are exercised.  Returns the [rows, cols] view."""
    rows, cols = arr2d.shape
    ld = cols if ld is None else ld
    g = Guard2D(rows, cols, dtype, ld, offset, f"input [{rows}, {cols}] ld {ld}")
    if rows and cols:
        g.t.copy_(to_dev(arr2d, dtype).view(rows, cols))
    return g.t


def empty_padded(rows, cols, dtype, ld=None, offset=0, fill=float("nan")):
    """An output view [rows, cols] filled with ``fill`` (row gaps and bands hold
    the sentinel).  Returns (view, guard)."""
    ld = cols if ld is None else ld
    g = Guard2D(rows, cols, dtype, ld, offset, f"output [{rows}, {cols}] ld {ld}")
    if rows and cols:
        g.t.fill_(fill)
    return g.t, g


class Guarded:
    """A 1-D output with sentinel bands before and after it (out-of-bounds write detector)."""

    SENTINEL = {torch.float32: -12345.5, torch.float16: -1234.0, torch.bfloat16: -1234.0,
                torch.int32: -77777}

    def __init__(self, n, dtype, fill=None):
        self.n = n
        s = self.SENTINEL[dtype]
        self.buf = torch.full((GUARD + n + GUARD,), s, dtype=dtype, device=DEV)
        self.t = self.buf[GUARD:GUARD + n]
        if fill is not None:
            self.t.fill_(fill)
        self.s = s

    def intact(self) -> bool:
        torch.cuda.synchronize()
        lo = self.buf[:GUARD]
        hi = self.buf[GUARD + self.n:]
        return bool((lo == self.s).all().item()) and bool((hi == self.s).all().item())


def pick_rows(n_rows, k, seed):
    """First, last and k random row indices (sorted, unique)."""
    g = np.random.default_rng(seed)
    idx = set([0, n_rows - 1]) | set(g.integers(0, n_rows, size=min(k, n_rows)).tolist())
    return np.array(sorted(idx), dtype=np.int64)


def chunked(fn, total, step, workers=16):
    """fn(start, stop) for consecutive chunks of [0, total), on a thread pool
    (the oracle's numpy work releases the GIL); results in chunk order."""
    from concurrent.futures import ThreadPoolExecutor

    starts = list(range(0, total, step))
    with ThreadPoolExecutor(max(1, min(workers, len(starts)))) as ex:
        return list(ex.map(lambda i: fn(i, min(i + step, total)), starts))
