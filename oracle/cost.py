"""Realized attention cost per (query block, KV chunk).  (Oracle: test infrastructure only.)

Split-KV page, Abstract: LPT balances the context KV chunks by their realized
attention cost, which is nonlinear and sample dependent under anchor sampling.
The pages give no unit; the reading used is the number of visible
(query, context key) pairs of one head:

    counts[b][c]  = B * #{ k in [c0, c1) : ctx_begin_b <= k < anchor_b }
    chunk_cost[c] = sum_b counts[b][c]

in int64.  The draft block's own keys are not a context chunk and carry no cost.
Here the count is taken by enumerating the keys one position at a time.
"""
from __future__ import annotations

import numpy as np

from .mask import visible_context


def chunk_costs(anchor, ctx_begin, block_size: int, chunk_start, chunk_len):
    """-> (counts int64 [n_blocks, n_chunks], chunk_cost int64 [n_chunks])."""
    nb, nc = len(anchor), len(chunk_start)
    counts = np.zeros((nb, nc), dtype=np.int64)
    for b in range(nb):
        lo, hi = visible_context(anchor, ctx_begin, b)
        for c in range(nc):
            keys = int(chunk_start[c]) + np.arange(int(chunk_len[c]), dtype=np.int64)
            seen = int(np.count_nonzero((keys >= lo) & (keys < hi)))
            counts[b, c] = block_size * seen
    chunk_cost = np.zeros(nc, dtype=np.int64)
    for b in range(nb):
        chunk_cost += counts[b]
    return counts, chunk_cost
