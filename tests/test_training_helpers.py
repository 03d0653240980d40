"""Host-side training helpers: the router-entropy schedule and the
load-balancing trend (CPU only)."""
import numpy as np
import pytest

from sparse_mixture_experts_capacity_amd.training import LoadBalanceTrend, router_entropy_coef


def test_entropy_schedule_high_early_low_late():
    total, high, low = 101, 0.5, 0.01
    vals = [router_entropy_coef(s, total, high, low) for s in range(total)]
    assert vals[0] == high and vals[-1] == pytest.approx(low, abs=1e-15)
    assert all(a >= b for a, b in zip(vals, vals[1:]))          # never rises
    assert vals[50] == pytest.approx((high + low) / 2)           # straight line
    assert router_entropy_coef(500, total, high, low) == pytest.approx(low)
    assert router_entropy_coef(-3, total, high, low) == high
    assert router_entropy_coef(0, 1, high, low) == low


def test_trend_slope_matches_least_squares():
    t = LoadBalanceTrend(window=50)
    assert t.slope() is None and t.last() is None
    rng = np.random.default_rng(0)
    ys = 2.0 - 0.01 * np.arange(80) + rng.normal(0, 0.002, 80)
    for y in ys:
        t.add(float(y))
    # only the last 50 steps count
    ref = np.polyfit(np.arange(30, 80), ys[30:], 1)[0]
    assert t.slope() == pytest.approx(ref, rel=1e-9)
    assert len(t) == 50 and t.summary()["steps"] == 80
    assert t.mean() == pytest.approx(float(np.mean(ys[30:])))


def test_trend_constant_and_exact_line():
    t = LoadBalanceTrend(window=10)
    for _ in range(12):
        t.add(1.0)                      # a balanced load: aux = 1 every step
    assert t.slope() == pytest.approx(0.0, abs=1e-15) and t.last() == 1.0
    u = LoadBalanceTrend(window=4)
    for s in range(4):
        u.add(3.0 - 0.5 * s)
    assert u.slope() == pytest.approx(-0.5)
    with pytest.raises(ValueError):
        LoadBalanceTrend(window=1)
