"""The CPU oracle against its pins (no GPU).  See tests/pins.py for what each pin is."""
import numpy as np
import pytest

import oracle
from pins import PINS

IMPL = {
    "weighted_sum": oracle.weighted_sum,
    "scaled_silu": oracle.scaled_silu,
    "softmax": oracle.softmax,
    "softmax_xent": oracle.softmax_xent,
    "norms": oracle.norms,
    "gather": oracle.gather,
}

CASES = [(op, name, fn, thr) for op, pins in PINS.items() for (name, fn, thr) in pins]


@pytest.mark.parametrize("op,name,fn,thr", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_oracle_pin(op, name, fn, thr):
    err = fn(IMPL[op])
    assert np.isfinite(err) and err <= thr, f"{op}/{name}: error {err:.3e} > {thr:.1e}"


def test_gradient_shapes_match_inputs():
    """The gradient has the shape of the thing it is the gradient of."""
    g = np.random.default_rng(0)
    x = g.standard_normal((7, 5))
    w = g.standard_normal(5)
    gx, gw = oracle.weighted_sum.bwd(g.standard_normal(7), x, w)
    assert gx.shape == x.shape and gw.shape == w.shape
    dx, dw = oracle.scaled_silu.bwd(g.standard_normal(11), g.standard_normal(11), 0.75)
    assert dx.shape == (11,) and np.ndim(dw) == 0
    y = oracle.softmax.fwd(x)
    assert oracle.softmax.bwd(x, y).shape == x.shape
    out = oracle.softmax_xent.fwd_bwd(x, np.array([0, 1, 2, 3, 4, 0, 1]), 1 / 7)
    assert out["dz"].shape == x.shape and out["row_lse"].shape == (7,)


def test_zero_rows():
    """Empty batches: empty outputs, zero parameter gradient, NaN mean loss."""
    x = np.zeros((0, 4))
    gx, gw = oracle.weighted_sum.bwd(np.zeros(0), x, np.ones(4))
    assert gx.shape == (0, 4) and np.all(gw == 0)
    _, dw = oracle.scaled_silu.bwd(np.zeros(0), np.zeros(0), 0.75)
    assert dw == 0
    out = oracle.softmax_xent.fwd_bwd(np.zeros((0, 3)), np.zeros(0, np.int64), 1.0)
    assert np.isnan(out["loss"]) and out["n_invalid"] == 0
