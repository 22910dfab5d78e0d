"""The block-sparse visibility rule.  (Oracle: test infrastructure only.)

Split-KV page, Abstract: anchor sampling builds compact draft queries, and the
draft queries cross-attend the context under a block-sparse mask.  The pages do
not spell the mask out; the reading used throughout is:

* each anchor owns one block of ``B`` draft queries (query rows ``b*B .. b*B+B-1``);
* every query of block ``b`` sees the context keys ``[ctx_begin_b, anchor_b)`` in
  packed (global) positions, where ``ctx_begin_b`` is the start of the block's
  own sample (0 for a single-sample context), i.e. its sample's keys strictly
  before the anchor;
* and, bidirectionally, the ``B`` keys of its own draft block, which are the draft
  tokens' own keys/values (``K_self``/``V_self`` rows ``b*B .. b*B+B-1``), not
  context positions.
"""
from __future__ import annotations

import numpy as np


def visible_context(anchor, ctx_begin, b: int):
    """Half-open packed range ``[lo, hi)`` of context keys visible to block ``b``."""
    return int(ctx_begin[b]), int(anchor[b])


def mask_error(anchor, ctx_begin, ctx_len: int) -> bool:
    """True when some block's range is not a valid interval of the context:
    ``ctx_begin < 0``, ``ctx_begin > anchor`` or ``anchor > ctx_len``."""
    for b in range(len(anchor)):
        lo, hi = visible_context(anchor, ctx_begin, b)
        if lo < 0 or lo > hi or hi > ctx_len:
            return True
    return False


def block_of_query(q: int, block_size: int) -> int:
    return q // block_size


def dense_mask(anchor, ctx_begin, block_size: int, ctx_len: int) -> np.ndarray:
    """Boolean [N_q, S + N_q] mask over (context keys, then all draft keys), built key by key.

    Only used by tests on tiny inputs: it spells out the rule one (query, key) pair at a time.
    """
    nb = len(anchor)
    nq = nb * block_size
    m = np.zeros((nq, ctx_len + nq), dtype=bool)
    for q in range(nq):
        b = block_of_query(q, block_size)
        lo, hi = visible_context(anchor, ctx_begin, b)
        for k in range(ctx_len):
            m[q, k] = lo <= k < hi
        for j in range(nq):
            m[q, ctx_len + j] = block_of_query(j, block_size) == b
    return m
