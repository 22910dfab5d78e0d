"""Longest-processing-time-first assignment of chunks to bins.  (Oracle: test infrastructure only.)

Split-KV page, Abstract: a cost-aware LPT strategy assigns context KV chunks to
context-parallel ranks by realized cost and reaches about 1% imbalance.  LPT is
Graham's rule: take the items longest first and give each to the least loaded
bin.  The pages fix neither ties nor the imbalance measure; the readings are:

* items in order of (cost descending, index ascending);
* each goes to the bin with (load ascending, index ascending);
* zero-cost items are placed like any other;
* makespan = max bin load, imbalance = makespan / (total / n_bins) - 1, and 0
  when the total is 0.
"""
from __future__ import annotations

import itertools


def lpt(cost, n_bins: int):
    """-> (bin_of list[int], loads list[int], makespan int, imbalance float)."""
    cost = [int(c) for c in cost]
    order = sorted(range(len(cost)), key=lambda i: (-cost[i], i))
    loads = [0] * n_bins
    bin_of = [-1] * len(cost)
    for i in order:
        j = min(range(n_bins), key=lambda t: (loads[t], t))
        bin_of[i] = j
        loads[j] += cost[i]
    makespan = max(loads) if loads else 0
    total = sum(cost)
    imbalance = makespan / (total / n_bins) - 1.0 if total > 0 else 0.0
    return bin_of, loads, makespan, imbalance


def lpt_makespan_opt(cost, n_bins: int) -> int:
    """Optimal makespan by enumerating every assignment (tiny instances only)."""
    cost = [int(c) for c in cost]
    best = None
    for assign in itertools.product(range(n_bins), repeat=len(cost)):
        loads = [0] * n_bins
        for c, j in zip(cost, assign):
            loads[j] += c
        m = max(loads)
        if best is None or m < best:
            best = m
    return best if best is not None else 0
