"""The tolerance rules of oracle.compare on hand-made values (no GPU)."""
import numpy as np
import pytest

from oracle.compare import combine, pointwise, reduced


def test_reduced_strict_rule():
    o = np.array([3.0, -4.0])                           # ||o|| = 5
    assert reduced(o * (1 + 0.9e-4), o).ok
    assert not reduced(o * (1 + 1.1e-4), o).ok
    # the sums of |terms| only report the condition number; they loosen nothing
    r = reduced(o * (1 + 1.1e-4), o, S=[300.0, 400.0])
    assert not r.ok and r.cond == pytest.approx(100.0) and r.rule == "rel-L2 1e-4"


def test_reduced_crafted_cancellation():
    o = np.array([2.0])
    g = np.array([2.0 + 5e-3])                          # 2.5e-3 relative: fails the strict rule
    assert not reduced(g, o, S=[1000.0]).ok
    r = reduced(g, o, S=[1000.0], crafted_cancellation=True)   # |g - o| <= 1e-5 * 1000
    assert r.ok and r.rule.startswith("abs 1e-5*S") and r.cond == pytest.approx(500.0)
    assert not reduced(g, o, S=[100.0], crafted_cancellation=True).ok
    with pytest.raises(ValueError):
        reduced(g, o, crafted_cancellation=True)


def test_reduced_nan_positions_must_match():
    assert reduced(np.array([np.nan, 1.0]), np.array([np.nan, 1.0])).ok
    assert not reduced(np.array([0.0, 1.0]), np.array([np.nan, 1.0])).ok


def test_combine_adds_counts():
    a = pointwise(np.array([1.0, 2.0], np.float32), np.array([1.0, 2.0]), "f32", name="a")
    b = pointwise(np.array([1.0, 3.0], np.float32), np.array([1.0, 2.0]), "f32", name="b")
    c = combine([a, b], "all")
    assert c.n == 4 and c.n_fail == 1 and not c.ok and c.max_rel == pytest.approx(0.5)
