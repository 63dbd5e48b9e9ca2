"""Comparison of HIP-path outputs with oracle values -- test infrastructure.

Tolerance rules (u = 2^-24, the fp32 unit roundoff):

* ``exact``      -- bitwise equality of the stored patterns.  Used where the
                    result is one exactly rounded operation of exact inputs
                    (the weighted-sum input gradient dy_i * w_j) and for
                    integers.
* ``pointwise``  -- for fp32 outputs: |g - o| <= 1e-5 * max(|o|, S), with S
                    the sum of the magnitudes of the terms that formed the
                    value (S = |o| for a value that is not a sum); values
                    that fp32 cannot hold to that precision (the subnormal
                    range and below) may differ by 2 fp32 ulp of o.
                    For fp16 / bf16 outputs: the ulp distance between the
                    stored result and the oracle rounded (once, directly) to
                    that dtype is at most 2; or, where the exact value is
                    cancellation-limited, |g - o| <= 2 ulp(o) + F with F a
                    floor derived per output from the fp32 arithmetic that
                    computes it (passed in by the caller).  How many
                    elements needed the floor is reported.
* ``reduced``    -- for parameter gradients and the mean loss:
                    ||g - o||_2 <= 1e-4 ||o||_2, always.  With S (the sums
                    of the magnitudes of the terms of each reduced value)
                    the condition number ||S||_2 / ||o||_2 is computed and
                    reported.  Only a test that builds a cancelling sum on
                    purpose (``crafted_cancellation=True``, its name says
                    so) may instead pass with |g - o| <= 1e-5 S element by
                    element, the fp32 accumulation bound for such a sum;
                    the report names the rule that passed.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import rounding

U32 = 2.0 ** -24


def _ordered16(bits: np.ndarray) -> np.ndarray:
    """Map 16-bit float patterns to integers that are consecutive in value order."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _bits(storage: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.asarray(storage, np.uint16)
    if dtype == "f16":
        return np.asarray(storage, np.float16).view(np.uint16)
    if dtype == "f32":
        return np.asarray(storage, np.float32).view(np.uint32)
    raise ValueError(dtype)


def _decode(storage: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (np.asarray(storage, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(storage, np.float16).astype(np.float64)
    return np.asarray(storage, np.float32).astype(np.float64)


@dataclass
class Report:
    name: str
    n: int = 0
    n_fail: int = 0
    n_floor: int = 0
    max_ulp: float = 0.0
    max_rel: float = 0.0
    worst: list = field(default_factory=list)
    rule: str = ""
    cond: float | None = None

    @property
    def ok(self) -> bool:
        return self.n_fail == 0

    def __str__(self) -> str:
        s = (f"{self.name}: n={self.n} fail={self.n_fail} floor_only={self.n_floor} "
             f"max_ulp={self.max_ulp:g} max_rel={self.max_rel:.3g}")
        if self.cond is not None:
            s += f" cond={self.cond:.3g}"
        if self.rule:
            s += f" rule={self.rule}"
        if self.worst:
            s += f" worst={self.worst[:3]}"
        return s


def exact(got_storage, ref_storage, dtype: str, name: str = "") -> Report:
    g = _bits(got_storage, dtype).reshape(-1)
    r = _bits(ref_storage, dtype).reshape(-1)
    rep = Report(name, n=g.size)
    bad = g != r
    rep.n_fail = int(np.count_nonzero(bad))
    if rep.n_fail:
        idx = np.nonzero(bad)[0][:5]
        rep.worst = [(int(i), int(g[i]), int(r[i])) for i in idx]
    return rep


def pointwise(got_storage, ref64, dtype: str, S=None, floor=None, name: str = "") -> Report:
    """See the module docstring.  ``S``: magnitude sums for fp32 outputs.
    ``floor``: per-element cancellation floor F for 16-bit outputs."""
    ref64 = np.asarray(ref64, np.float64).reshape(-1)
    got = _decode(got_storage, dtype).reshape(-1)
    rep = Report(name, n=got.size)
    if got.size == 0:
        return rep
    nan_ref = np.isnan(ref64)
    nan_bad = nan_ref != np.isnan(got)
    fin = ~nan_ref & ~np.isnan(got)
    if dtype == "f32":
        scale = np.abs(ref64) if S is None else np.maximum(np.abs(ref64), np.asarray(S, np.float64).reshape(-1))
        err = np.abs(got - ref64)
        with np.errstate(invalid="ignore", over="ignore"):
            floor32 = 2.0 * rounding.ulp(rounding.round_to(np.where(np.isfinite(ref64), ref64, 0.0), "f32"), "f32")
        err = np.where(err <= floor32, 0.0, err)
        with np.errstate(invalid="ignore", divide="ignore"):
            rel = np.where(scale > 0, err / scale, np.where(err > 0, np.inf, 0.0))
        inf_same = np.isinf(ref64) & (got == ref64)
        rel = np.where(inf_same, 0.0, rel)
        bad = (fin & (rel > 1e-5)) | nan_bad
        rep.max_rel = float(np.max(rel[fin])) if fin.any() else 0.0
    else:
        r16 = rounding.round_to(ref64, dtype)
        rbits = _bits(rounding.to_storage(r16, dtype), dtype)
        gbits = _bits(got_storage, dtype).reshape(-1)
        ud = np.abs(_ordered16(gbits) - _ordered16(rbits)).astype(np.float64)
        strict = ud <= 2
        if floor is not None:
            F = np.asarray(floor, np.float64).reshape(-1)
            lim = 2.0 * rounding.ulp(r16, dtype) + F
            with np.errstate(invalid="ignore"):
                floor_ok = np.abs(got - ref64) <= lim
        else:
            floor_ok = np.zeros_like(strict)
        passed = strict | floor_ok
        bad = (fin & ~passed) | nan_bad
        rep.n_floor = int(np.count_nonzero(fin & ~strict & floor_ok))
        rep.max_ulp = float(np.max(ud[fin])) if fin.any() else 0.0
        with np.errstate(invalid="ignore", divide="ignore"):
            rel = np.abs(got - ref64) / np.abs(ref64)
        rep.max_rel = float(np.nanmax(np.where(fin & (ref64 != 0), rel, 0.0)))
    rep.n_fail = int(np.count_nonzero(bad))
    if rep.n_fail:
        idx = np.nonzero(bad)[0][:5]
        rep.worst = [(int(i), float(got[i]), float(ref64[i])) for i in idx]
    return rep


def reduced(got, ref64, name: str = "", S=None, crafted_cancellation: bool = False) -> Report:
    """Parameter gradients and the mean loss: ||g - o||_2 <= 1e-4 ||o||_2.

    ``S``: per-value sums of |terms| (same shape as ``ref64``); gives the
    condition number ||S||_2 / ||o||_2 that the report carries.
    ``crafted_cancellation``: for tests whose inputs cancel on purpose only;
    then |g - o| <= 1e-5 S element by element also passes (needs S).
    """
    g = np.asarray(got, np.float64).reshape(-1)
    r = np.asarray(ref64, np.float64).reshape(-1)
    rep = Report(name, n=g.size, rule="rel-L2 1e-4")
    if crafted_cancellation and S is None:
        raise ValueError("crafted_cancellation needs S")
    if S is not None:
        S = np.asarray(S, np.float64).reshape(-1)
        nr_all = float(np.linalg.norm(r[~np.isnan(r)])) if r.size else 0.0
        ns = float(np.linalg.norm(S))
        rep.cond = ns / nr_all if nr_all > 0 else (0.0 if ns == 0 else np.inf)
    if g.size == 0:
        return rep
    if np.any(np.isnan(r)) or np.any(np.isnan(g)):
        rep.n_fail = int(np.count_nonzero(np.isnan(r) != np.isnan(g)))
        m = ~np.isnan(r) & ~np.isnan(g)
        g, r = g[m], r[m]
        if S is not None:
            S = S[m]
        if g.size == 0:
            return rep
    nr = float(np.linalg.norm(r))
    err = float(np.linalg.norm(g - r))
    rel = err / nr if nr > 0 else (0.0 if err == 0 else np.inf)
    rep.max_rel = rel
    if rel > 1e-4:
        if crafted_cancellation and np.all(np.abs(g - r) <= 1e-5 * S):
            rep.n_floor = g.size
            rep.rule = "abs 1e-5*S (crafted cancellation)"
        else:
            rep.n_fail += 1
            rep.worst = [(err, nr)]
    return rep


def combine(reps, name: str) -> Report:
    """One report for an output compared in chunks: counts add up, maxima
    and the first few worst cases carry over."""
    out = Report(name)
    for r in reps:
        out.n += r.n
        out.n_fail += r.n_fail
        out.n_floor += r.n_floor
        out.max_ulp = max(out.max_ulp, r.max_ulp)
        out.max_rel = max(out.max_rel, r.max_rel)
        if r.worst and len(out.worst) < 5:
            out.worst.extend(r.worst[:5 - len(out.worst)])
    return out
