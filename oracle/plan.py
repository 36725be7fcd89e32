"""ORACLE -- test infrastructure only (tests, the smoke check and the CPU leg
of the benchmark may use it; the product library never does).

Per-request buffer sizing, written out as its definition.  The Spin summary
(gist.science 2604.26837, section 2B, buffer elasticity) sizes each
request's device buffer dynamically: mandatory pages, needed by the current
step, and buffer pages, kept for temporal locality, with a planner that
weighs per-request throughput against contention across the system.  The
page gives no formula; the reading taken is:

  * mandatory slots of unit u = demand[u], the size of its next union, which
    must lie in [1, S];
  * if the mandatory slots of all units exceed the budget, the plan does not
    fit (the scheduler must admit fewer requests): None;
  * the spare budget (budget minus all mandatory slots) is shared in
    proportion to reuse[u] + 1, where reuse[u] counts the unit's recent hits,
    rounded down: extra[u] = floor(spare * (reuse[u] + 1) / sum(reuse + 1));
  * capacity[u] = min(S, demand[u] + extra[u]).
"""
from __future__ import annotations

import numpy as np


def plan_capacity(demand, reuse, budget: int, S: int):
    demand = [int(x) for x in demand]
    reuse = [int(x) for x in reuse]
    assert len(demand) == len(reuse)
    if any(d < 1 or d > S for d in demand) or any(r < 0 for r in reuse):
        raise ValueError("demand outside [1, S] or negative reuse")
    mandatory = sum(demand)
    if mandatory > budget:
        return None
    spare = budget - mandatory
    weights = [r + 1 for r in reuse]
    total = sum(weights)
    return np.array([min(S, d + (spare * wgt) // total) for d, wgt in zip(demand, weights)],
                    dtype=np.int32)
