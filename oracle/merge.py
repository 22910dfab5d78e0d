"""Exact merge of partial (O, LSE) pairs.  (Oracle: test infrastructure only.)

Split-KV page, Abstract: the method is exact and moves only query-sized tensors
per layer.  The pages print no merge formula; the one that makes a split of the
keys exact is the log-sum-exp combination of normalized partials:

    M   = max_p LSE_p
    LSE = M + log sum_p exp(LSE_p - M)
    O   = sum_p exp(LSE_p - LSE) * O_p

taken over the partials in ascending slot order.  A partial with LSE_p = -inf
(no visible key) is skipped, never multiplied, so its O_p is never read; when all
partials of a row are -inf the merged row is (O = 0, LSE = -inf).
"""
from __future__ import annotations

import numpy as np


def lse_merge(o_parts, lse_parts):
    """o_parts [P, R, d], lse_parts [P, R] -> (O [R, d], LSE [R]) in float64."""
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    n_parts, n_rows = lse_parts.shape
    d = o_parts.shape[-1]
    m = np.full(n_rows, -np.inf)
    for p in range(n_parts):
        m = np.maximum(m, lse_parts[p])
    live = m > -np.inf
    acc = np.zeros(n_rows)
    for p in range(n_parts):
        fin = lse_parts[p] > -np.inf
        acc[fin] += np.exp(lse_parts[p][fin] - m[fin])
    lse = np.full(n_rows, -np.inf)
    lse[live] = m[live] + np.log(acc[live])
    o = np.zeros((n_rows, d))
    for p in range(n_parts):
        fin = lse_parts[p] > -np.inf
        w = np.exp(lse_parts[p][fin] - lse[fin])
        o[fin] += w[:, None] * np.asarray(o_parts[p], dtype=np.float64)[fin]
    return o, lse
