"""The five reference workloads (shapes, dtypes, value distributions, seeds).

Each workload is named by what it is.  ``sigma`` is the standard deviation
of the normal draw.  Seeds are ``1000 + k`` for the k-th workload; the
streams of :mod:`synth` separate x, w, dy and targets.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    op: str                 # "weighted_sum" | "scaled_silu" | "softmax" | "softmax_xent" | "gather_rows"
    dtype: str              # activation storage dtype
    shape: tuple            # x / logits shape
    seed: int
    sigma_x: float
    sigma_dy: float = 1.0
    w_dtype: str = "f32"
    sigma_w: float = 1.0
    w_value: float | None = None     # scalar weight given as a constant
    rows_per_tile: int = 0           # 0 = library's automatic choice
    extra: dict = field(default_factory=dict)


WS_SMALL = Workload("weighted_sum_f32_100x64", "weighted_sum", "f32", (100, 64), 1000,
                    sigma_x=1.0, sigma_dy=1.0, w_dtype="f32", sigma_w=1.0, rows_per_tile=32)
SILU_16M = Workload("scaled_silu_f16_n16777216", "scaled_silu", "f16", (1 << 24,), 1001,
                    sigma_x=2.0, sigma_dy=1.0, w_value=0.75)
WS_LARGE = Workload("weighted_sum_bf16_1048576x256", "weighted_sum", "bf16", (1 << 20, 256), 1002,
                    sigma_x=1.0, sigma_dy=1.0, w_dtype="bf16", sigma_w=0.1)
SOFTMAX = Workload("softmax_bf16_32768x4096", "softmax", "bf16", (32768, 4096), 1003,
                   sigma_x=3.0, sigma_dy=1.0)
XENT = Workload("softmax_xent_bf16_16384x32000", "softmax_xent", "bf16", (16384, 32000), 1004,
                sigma_x=2.0, extra={"grad_scale": 1.0 / 16384})

# Embedding lookup (gather) and its scatter-add backward: 16384 tokens with
# Zipf(1.2) ids over a 32000-row table of 4096-wide bf16 rows.
EMBED = Workload("gather_rows_bf16_16384x32000x4096", "gather_rows", "bf16", (16384, 4096), 1005,
                 sigma_x=1.0, extra={"V": 32000, "zipf_a": 1.2})

ALL = (WS_SMALL, SILU_16M, WS_LARGE, SOFTMAX, XENT, EMBED)
BY_NAME = {w.name: w for w in ALL}
