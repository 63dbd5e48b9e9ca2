"""The oracle's direct fp64 -> dtype rounding against brute force and library casts (no GPU).

* bf16 and f16: every finite value of the format is enumerated from its bit
  patterns; the nearest one is found by search, ties going to the even bit
  pattern, and the overflow threshold 2^(emax+1) counting as an even
  neighbour that maps to infinity.  Exact comparisons use Fraction.
* f32: numpy's float64 -> float32 cast (IEEE round to nearest even).
* f16: numpy's float64 -> float16 cast (rounds directly from double).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle.rounding import FORMATS, round_to, to_storage, ulp


def _all_values(dtype):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if dtype == "bf16":
        v = synth.to_f64(bits, "bf16")
    else:
        v = bits.view(np.float16).astype(np.float64)
    return bits, v


def _nonneg_grid(dtype):
    """Sorted non-negative finite values with their bit patterns, plus the overflow point."""
    bits, v = _all_values(dtype)
    sel = np.isfinite(v) & (np.signbit(v) == 0)
    vals, pats = v[sel], bits[sel].astype(np.int64)
    order = np.argsort(vals)
    vals, pats = vals[order], pats[order]
    _, _, emax = FORMATS[dtype]
    vals = np.append(vals, 2.0 ** (emax + 1))
    pats = np.append(pats, pats[-1] + 1)           # even pattern beyond the largest finite
    return vals, pats


def _test_values(dtype, n, seed):
    g = np.random.default_rng(seed)
    p, emin, emax = FORMATS[dtype]
    e = g.integers(emin - p - 3, emax + 2, size=n)
    v = np.ldexp(1.0 + g.random(n), e)
    grid, _ = _nonneg_grid(dtype)
    mids = (grid[:-1] + grid[1:]) / 2                 # exact ties (exact in fp64)
    pick = g.choice(mids, size=n // 4)
    nudged = np.concatenate([pick, np.nextafter(pick, 0), np.nextafter(pick, np.inf)])
    v = np.concatenate([v, nudged, grid[:-1], [0.0, 2.0 ** (emax + 1) * 4]])
    signs = np.where(g.random(v.size) < 0.5, -1.0, 1.0)
    return v * signs


def _brute(dtype, v):
    grid, pats = _nonneg_grid(dtype)
    a = np.abs(v)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, grid.size - 1)
    lo = np.clip(hi - 1, 0, grid.size - 1)
    dlo = a - grid[lo]
    dhi = grid[hi] - a
    choose_hi = (dhi < dlo) | ((dhi == dlo) & (pats[hi] % 2 == 0))
    choose_hi |= a == grid[hi]
    r = np.where(choose_hi, grid[hi], grid[lo])
    r = np.where(r >= grid[-1], np.inf, r)
    return np.copysign(r, v)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_round_brute_force(dtype):
    v = _test_values(dtype, 200_000, 1)
    got = round_to(v, dtype)
    ref = _brute(dtype, v)
    bad = ~((got == ref) | (np.isnan(got) & np.isnan(ref)))
    assert not bad.any(), (v[bad][:5], got[bad][:5], ref[bad][:5])
    assert np.array_equal(np.signbit(got), np.signbit(ref))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_round_exact_fraction_sample(dtype):
    """A sample re-checked with exact rational distances (no floating point at all)."""
    v = _test_values(dtype, 400, 2)[:1500]
    grid, pats = _nonneg_grid(dtype)
    got = round_to(v, dtype)
    for x, r in zip(v, got):
        a = Fraction(abs(float(x)))
        i = int(np.searchsorted(grid, float(abs(x))))
        cands = [j for j in (i - 1, i) if 0 <= j < grid.size]
        best = min(cands, key=lambda j: (abs(Fraction(float(grid[j])) - a), pats[j] % 2))
        ref = grid[best]
        ref = np.inf if ref >= grid[-1] else ref
        assert abs(r) == ref, (x, r, ref)


def test_round_f32_matches_numpy_cast():
    g = np.random.default_rng(3)
    e = g.integers(-160, 130, size=500_000)
    v = np.ldexp(1.0 + g.random(500_000), e) * np.where(g.random(500_000) < 0.5, -1, 1)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32).astype(np.float64)
    got = round_to(v, "f32")
    assert np.array_equal(got, ref)


def test_round_f16_matches_numpy_cast():
    v = _test_values("f16", 300_000, 4)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).astype(np.float64)
    got = round_to(v, "f16")
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_round_trip_all_patterns(dtype):
    """Every representable value rounds to itself and encodes to its own bit pattern."""
    bits, v = _all_values(dtype)
    fin = np.isfinite(v)
    r = round_to(v, dtype)
    assert np.array_equal(r[fin], v[fin])
    enc = synth.bits16(to_storage(r[fin], dtype), dtype)
    assert np.array_equal(enc, bits[fin])
    assert np.all(np.isnan(r[np.isnan(v)]))
    assert np.array_equal(r[np.isinf(v)], v[np.isinf(v)])


def test_special_values_pass_through():
    v = np.array([0.0, -0.0, np.inf, -np.inf, np.nan])
    for dt in ("f32", "f16", "bf16"):
        r = round_to(v, dt)
        assert r[0] == 0 and not np.signbit(r[0]) and r[1] == 0 and np.signbit(r[1])
        assert r[2] == np.inf and r[3] == -np.inf and np.isnan(r[4])


def test_ulp_spacing():
    assert ulp(np.array([1.0]), "bf16")[0] == 2.0 ** -7
    assert ulp(np.array([1.0]), "f16")[0] == 2.0 ** -10
    assert ulp(np.array([1.5]), "f32")[0] == 2.0 ** -23
    assert ulp(np.array([0.0]), "f16")[0] == 2.0 ** -24          # smallest subnormal
    assert ulp(np.array([2.0 ** -130]), "bf16")[0] == 2.0 ** -133
