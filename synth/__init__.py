"""Seeded synthetic inputs for the VJP ops.

This module is shared by the CPU oracle checks, the GPU parity tests, the
benchmark and the smoke check.  It holds random draws, storage-format
conversion (fp64 <-> fp32 / fp16 / bf16 bit patterns) and the workload
table -- none of the arithmetic of the ops themselves.

Storage convention: an array in dtype ``"f32"`` is a numpy float32 array,
``"f16"`` a numpy float16 array, ``"bf16"`` a numpy uint16 array holding the
raw bfloat16 bit patterns (numpy has no bfloat16 type).

Random draws: PCG64 seeded with ``[seed, stream]`` through numpy's
SeedSequence; normals come from numpy's ``standard_normal`` in float32,
are scaled by sigma (sigma is the standard deviation) and rounded to the
storage dtype with round-to-nearest-even (torch's float32 -> bfloat16 cast,
numpy's float32 -> float16 cast).  Integer targets come from numpy's
``integers`` (uniform on ``[0, classes)``).
"""
from __future__ import annotations

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ITEMSIZE = {"f32": 4, "f16": 2, "bf16": 2}

# Streams of one workload seed (one independent generator per input tensor).
STREAM_X, STREAM_W, STREAM_DY, STREAM_TARGETS = 0, 1, 2, 3


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def f32_to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the storage dtype (RNE)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(a).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown dtype {dtype!r}")


def normal(shape, sigma: float, dtype: str, seed: int, stream: int) -> np.ndarray:
    """sigma * N(0, 1) drawn in float32, stored as ``dtype``."""
    g = rng(seed, stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(sigma)
    return f32_to_storage(a, dtype)


def targets(rows: int, classes: int, seed: int, stream: int = STREAM_TARGETS) -> np.ndarray:
    """Uniform int32 class indices in [0, classes)."""
    return rng(seed, stream).integers(0, classes, size=rows, dtype=np.int64).astype(np.int32)


STREAM_INDEX = 4


def zipf_indices(M: int, V: int, seed: int, a: float = 1.2, stream: int = STREAM_INDEX) -> np.ndarray:
    """M int32 row indices in [0, V) with a Zipf(a) rank distribution (a few
    rows drawn very often, as token ids in text are); ranks are mapped to rows
    through a seeded permutation so frequent rows are spread over the table."""
    g = rng(seed, stream)
    ranks = np.minimum(g.zipf(a, size=M), V) - 1
    perm = g.permutation(V) if V > 0 else np.zeros(0, np.int64)
    return perm[ranks].astype(np.int32) if V > 0 else np.zeros(M, np.int32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact value of every stored element as float64."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        with np.errstate(invalid="ignore"):
            return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits16(a: np.ndarray, dtype: str) -> np.ndarray:
    """Raw 16-bit patterns of an f16 or bf16 storage array."""
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).view(np.uint16)
    if dtype == "bf16":
        return np.asarray(a, dtype=np.uint16)
    raise ValueError(f"{dtype!r} is not a 16-bit format")


# --- torch glue (device memory only) -------------------------------------------

def torch_dtype(dtype: str):
    import torch

    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_torch(a: np.ndarray, dtype: str, device="cpu"):
    """Storage array -> torch tensor of the matching dtype (bit-for-bit)."""
    import torch

    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(a.astype(np.float16, copy=False))
    elif dtype == "f32":
        t = torch.from_numpy(a.astype(np.float32, copy=False))
    else:
        raise ValueError(dtype)
    return t.to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    """torch tensor -> storage array (bit-for-bit copy to the host)."""
    import torch

    t = t.detach().contiguous().cpu()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "f16":
        return t.numpy().astype(np.float16, copy=True)
    if dtype == "f32":
        return t.numpy().astype(np.float32, copy=True)
    raise ValueError(dtype)


def normal_device(shape, sigma: float, dtype: str, seed: int, stream: int, device):
    """sigma * N(0, 1) drawn directly on a device with torch's seeded generator.

    Used where only throughput is measured (the values never meet the
    oracle); parity inputs always come from :func:`normal`.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(stream))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(float(sigma))
    return t.to(torch_dtype(dtype))


def targets_device(rows: int, classes: int, seed: int, device, stream: int = STREAM_TARGETS):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(stream))
    return torch.randint(0, classes, (rows,), generator=g, device=device, dtype=torch.int32)
