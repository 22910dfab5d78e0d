"""Static chunk placements the pages compare LPT against.  (Oracle: test infrastructure only.)

Split-KV page, Figures & tables (the CP comparison table, load-balancing column):
Split-KV balances context KV chunks with cost-aware LPT, Ring Attention with a
zigzag layout, and RingX does no balancing.  The pages give the strategies' names
only; the readings, for chunks i = 0 .. n - 1 in context order and P ranks:

* contiguous (no balancing): the chunks form P runs of consecutive chunks, run r
  holding chunks i with floor(i * P / n) = r;
* zigzag: the chunks form 2P runs the same way, and rank r holds runs r and
  2P - 1 - r (one early and one late part of the context);
* round-robin: chunk i goes to rank i mod P.

Loads, makespan and imbalance are measured as for LPT (``oracle.lpt``).
"""
from __future__ import annotations


def _measure(cost, bin_of, n_bins):
    loads = [0] * n_bins
    for i, b in enumerate(bin_of):
        loads[b] += int(cost[i])
    makespan = max(loads) if loads else 0
    total = sum(int(c) for c in cost)
    imbalance = makespan / (total / n_bins) - 1.0 if total > 0 else 0.0
    return bin_of, loads, makespan, imbalance


def contiguous(cost, n_bins: int):
    """-> (bin_of, loads, makespan, imbalance) for P runs of consecutive chunks."""
    n = len(cost)
    return _measure(cost, [i * n_bins // n for i in range(n)], n_bins)


def zigzag(cost, n_bins: int):
    """-> (bin_of, loads, makespan, imbalance): rank r holds runs r and 2P - 1 - r of 2P."""
    n = len(cost)
    bin_of = []
    for i in range(n):
        run = i * 2 * n_bins // n
        bin_of.append(run if run < n_bins else 2 * n_bins - 1 - run)
    return _measure(cost, bin_of, n_bins)


def round_robin(cost, n_bins: int):
    """-> (bin_of, loads, makespan, imbalance) for chunk i on rank i mod P."""
    return _measure(cost, [i % n_bins for i in range(len(cost))], n_bins)
