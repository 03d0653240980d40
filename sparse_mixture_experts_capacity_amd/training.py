"""Training-side helpers around the router: the entropy coefficient's
schedule and the load-balancing trend.  Host logic only; the gradients
themselves come from ``moe_router_backward``.

[Routing guide] "MoE routing, fully explained" (allinfo.ai.kr), "Plain
explanation" para 4: the router's entropy is kept high early in training
(tokens explore many experts) and lowered later (each token commits to its
experts); "Key insights" item 3 lists the load-balancing loss's trend among
the quantities to watch.
"""
from __future__ import annotations

from collections import deque
from typing import Deque, Optional


def router_entropy_coef(step: int, total_steps: int, high: float, low: float) -> float:
    """Coefficient of the mean router entropy in the loss at ``step`` of
    ``total_steps``: ``high`` at the first step, falling linearly to ``low``
    at the last (and held there after it).  The page gives only the
    direction (high early, lower later); a straight line is the plainest
    schedule with that shape."""
    if total_steps <= 1:
        return float(low)
    s = min(max(int(step), 0), total_steps - 1)
    frac = s / (total_steps - 1)
    return float(high + (low - high) * frac)


class LoadBalanceTrend:
    """The load-balancing loss over recent training steps.

    ``add(aux)`` records one step's auxiliary loss (``stats["aux_loss"]`` of
    the forward).  ``slope()`` is the least-squares slope of the last
    ``window`` values against their step numbers (per step): negative while
    the load evens out, near zero once it has settled.  aux is 1 for a
    perfectly balanced load and E at full concentration, so ``last()`` and
    ``mean()`` read on that scale."""

    def __init__(self, window: int = 100):
        if window < 2:
            raise ValueError("window must be at least 2")
        self.window = int(window)
        self._vals: Deque[float] = deque(maxlen=self.window)
        self._steps: Deque[int] = deque(maxlen=self.window)
        self._n = 0

    def add(self, aux_loss: float) -> None:
        self._vals.append(float(aux_loss))
        self._steps.append(self._n)
        self._n += 1

    def __len__(self) -> int:
        return len(self._vals)

    def last(self) -> Optional[float]:
        return self._vals[-1] if self._vals else None

    def mean(self) -> Optional[float]:
        return sum(self._vals) / len(self._vals) if self._vals else None

    def slope(self) -> Optional[float]:
        n = len(self._vals)
        if n < 2:
            return None
        xs, ys = list(self._steps), list(self._vals)
        mx = sum(xs) / n
        my = sum(ys) / n
        sxx = sum((a - mx) ** 2 for a in xs)
        sxy = sum((a - mx) * (b - my) for a, b in zip(xs, ys))
        return sxy / sxx

    def summary(self) -> dict:
        return dict(steps=self._n, window=len(self._vals), last=self.last(),
                    mean=self.mean(), slope=self.slope())
