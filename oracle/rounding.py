"""Direct fp64 -> {fp32, fp16, bf16} rounding, round to nearest, ties to even.

Test infrastructure (see the package docstring).

A binary format with p significand bits and minimum normal exponent emin
represents, in the binade [2^E, 2^(E+1)) with E >= emin, exactly the
multiples of 2^(E-p+1); below 2^emin (subnormals) the spacing stays
2^(emin-p+1).  Rounding to nearest even is therefore ``rint(v / q) * q``
with q that spacing (``np.rint`` rounds halves to even; dividing by a power
of two is exact).  A result whose magnitude reaches 2^(emax+1) overflows to
infinity.  Zeros keep their sign, NaN and infinities pass through.  No
flush-to-zero anywhere.
"""
from __future__ import annotations

import numpy as np

# dtype -> (significand bits p incl. the implicit bit, emin, emax)
FORMATS = {
    "f32": (24, -126, 127),
    "f16": (11, -14, 15),
    "bf16": (8, -126, 127),
}


def round_to(v, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype``; returns float64 holding the rounded values."""
    p, emin, emax = FORMATS[dtype]
    v = np.array(v, dtype=np.float64, copy=True)
    flat = v.reshape(-1)
    sel = np.isfinite(flat) & (flat != 0.0)
    x = flat[sel]
    _, e = np.frexp(x)                      # x = m * 2**e with 0.5 <= |m| < 1
    E = np.maximum(e - 1, emin)             # binade exponent, clamped for subnormals
    q = np.ldexp(np.ones_like(x), E - (p - 1))
    r = np.rint(x / q) * q
    over = np.abs(r) >= np.ldexp(1.0, emax + 1)
    r[over] = np.copysign(np.inf, r[over])
    flat[sel] = r
    return v


def to_storage(v_rounded, dtype: str) -> np.ndarray:
    """Values already rounded by :func:`round_to` -> storage array (exact)."""
    v = np.asarray(v_rounded, dtype=np.float64)
    if dtype == "f32":
        return v.astype(np.float32)
    if dtype == "f16":
        return v.astype(np.float16)
    if dtype == "bf16":
        return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(dtype)


def ulp(v_rounded, dtype: str) -> np.ndarray:
    """Spacing of ``dtype`` at each (already rounded) value: 2^(E-p+1)."""
    p, emin, _ = FORMATS[dtype]
    v = np.asarray(v_rounded, dtype=np.float64)
    a = np.abs(np.where(np.isfinite(v), v, 0.0))
    _, e = np.frexp(np.where(a == 0.0, 1.0, a))
    E = np.where(a == 0.0, emin, np.maximum(e - 1, emin))
    return np.ldexp(np.ones_like(a), E - (p - 1))
