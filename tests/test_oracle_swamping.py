"""The scaled-SiLU page's bf16 swamping example, against the oracle's fp64 dw (no GPU).

32,768 contributions of about 1e-3 (tests/golden/swamping_example.json): the
oracle's dw equals the exactly rounded sum (math.fsum); a running sum kept in
bf16 stalls once it passes ~1 and misses by far more than 10 %; an fp32
running sum keeps the page's ~7 digits.
"""
import math

import numpy as np

import oracle
from oracle.rounding import round_to
from pins import golden


def _crafted(n, mag):
    # dy * x * sigmoid(x) ~ mag for every element: x = 4 (sigmoid ~ 0.982), dy = mag / (x s)
    x = np.full(n, 4.0)
    s = oracle.scaled_silu.sigmoid(x)
    g = np.random.default_rng(0)
    dy = mag * (1.0 + 0.1 * g.standard_normal(n)) / (x * s)
    return dy, x


def test_swamping_example():
    case = golden("swamping_example.json")
    n, mag = case["contributions"], case["magnitude"]
    dy, x = _crafted(n, mag)
    terms = dy * x * oracle.scaled_silu.sigmoid(x)
    _, dw = oracle.scaled_silu.bwd(dy, x, 0.75)
    exact = math.fsum(terms)
    assert abs(dw - exact) <= 1e-12 * abs(exact)
    assert 30.0 < exact < 36.0

    acc_bf16 = 0.0
    acc_f32 = np.float32(0.0)
    for t in terms:
        acc_bf16 = float(round_to(np.array([acc_bf16 + float(round_to(np.array([t]), "bf16")[0])]), "bf16")[0])
        acc_f32 = np.float32(acc_f32 + np.float32(t))
    assert abs(acc_bf16 - exact) / exact > 0.10          # bf16 accumulator fails
    digits_f32 = -math.log10(abs(float(acc_f32) - exact) / exact)
    assert digits_f32 >= case["fp32_digits_kept"] - 2    # fp32 keeps ~5-7 digits over 32k terms
