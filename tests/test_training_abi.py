"""The training side of the router through the C ABI (host only, no GPU):
the router-entropy schedule and the load-balancing trend, each against the
oracle's own functions (which tests/pins.py pins to numpy.polyfit, closed
forms and routing batches of shrinking skew)."""
import math

import numpy as np
import pytest

import oracle.oracle as O
import sparse_mixture_experts_capacity_amd as moe


@pytest.mark.parametrize("total,high,low", [(101, 0.5, 0.01), (2, 1.0, 0.0), (7, 0.0, 0.3),
                                            (1000, 1e-3, 1e-5), (1, 0.5, 0.1)])
def test_entropy_coef_matches_oracle(total, high, low):
    for step in [-3, 0, 1, total // 2, total - 2, total - 1, total, 10 * total]:
        got = moe.moe_entropy_coef(step, total, high, low)
        ref = O.entropy_schedule(step, total, high, low)
        assert abs(got - ref) <= 1e-15 * max(1.0, abs(ref)), (step, got, ref)
    assert math.isnan(moe.moe_entropy_coef(0, 10, float("inf"), 0.0))


@pytest.mark.parametrize("n", [2, 3, 5, 50, 1000])
def test_lb_trend_matches_oracle(n):
    r = np.random.default_rng(n)
    v = 1.0 + np.abs(r.standard_normal(n)) * 0.3 - 0.001 * np.arange(n)
    slope, mean = moe.moe_lb_trend(v)
    ref = O.load_balance_trend(list(v))
    assert abs(slope - ref["slope"]) <= 1e-12 * max(1.0, abs(ref["slope"]))
    assert abs(mean - ref["mean"]) <= 1e-14


def test_lb_trend_errors():
    with pytest.raises(moe.MoeError) as e:
        moe.moe_lb_trend([1.0])
    assert e.value.code == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError):
        moe.moe_lb_trend([1.0, float("nan"), 2.0])


def test_window_keeps_the_last_steps():
    t = moe.LoadBalanceTrend(window=50)
    assert t.slope() is None and t.last() is None
    ys = 2.0 - 0.01 * np.arange(80)
    for y in ys:
        t.add(float(y))
    assert len(t) == 50 and t.steps == 80 and t.last() == ys[-1]
    assert t.slope() == pytest.approx(O.load_balance_trend(list(ys[30:]))["slope"], rel=1e-12)
    assert t.mean() == pytest.approx(float(np.mean(ys[30:])), rel=1e-14)
    with pytest.raises(ValueError):
        moe.LoadBalanceTrend(window=1)
