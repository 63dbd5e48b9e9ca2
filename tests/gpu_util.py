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


def padded(arr2d, dtype, ld=None, offset=0):
    """Upload a [rows, cols] storage array into a device buffer with row stride
    ``ld`` (>= cols) starting ``offset`` elements into the allocation, so that
    leading dimensions and base alignments other than the natural ones are
    exercised.  Returns the [rows, cols] view."""
    rows, cols = arr2d.shape
    ld = cols if ld is None else ld
    total = offset + max(rows - 1, 0) * ld + cols + 8
    buf = torch.zeros(total, dtype=synth.torch_dtype(dtype), device=DEV)
    view = buf.as_strided((rows, cols), (ld, 1), offset)
    if rows and cols:
        view.copy_(to_dev(arr2d, dtype))
    return view


def empty_padded(rows, cols, dtype, ld=None, offset=0, fill=float("nan")):
    ld = cols if ld is None else ld
    total = offset + max(rows - 1, 0) * ld + cols + 8
    buf = torch.full((total,), fill, dtype=synth.torch_dtype(dtype), device=DEV)
    return buf.as_strided((rows, cols), (ld, 1), offset), buf


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
