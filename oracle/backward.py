"""Gradients of masked softmax attention.  (Oracle: test infrastructure only.)

The training workload needs dQ, dK, dV of O = softmax(Q K^T / sqrt(d)) V (the
attention formula on the Flash-dLLM page, "Method 1") under the draft-block
mask.  The Split-KV page (Abstract) trains drafters with this attention but
prints no backward; the gradient below is the analytic one of the unchunked
attention, written per query row r = (q, h) and visible key k:

    P_rk  = exp(s_rk - LSE_r)
    D_r   = sum_i dO_ri * O_ri
    dP_rk = dO_r . v_k
    dS_rk = P_rk * (dP_rk - D_r)
    dQ_r += scale * dS_rk * k_k
    dK_k += scale * dS_rk * q_r      (summed over the query heads of k's KV head)
    dV_k += P_rk * dO_r

with (O, LSE) the merged (unchunked) forward results.  When only some chunks are
local (one context-parallel rank), the same formulas restricted to the local keys
give that rank's dK/dV exactly and its share of dQ; the shares over all ranks sum
to the full dQ.  The draft block's own keys take dK_self/dV_self.
"""
from __future__ import annotations

import numpy as np

from .attention import chunk_offsets, default_scale
from .mask import visible_context


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attention_backward(q, k_loc, v_loc, k_self, v_self, anchor, ctx_begin, block_size: int,
                       chunk_start, chunk_len, d_o, o, lse, with_self: bool = True,
                       scale: float = None, groups=None):
    """-> dq [N_q, H_q, d], dk [n_loc, H_kv, d], dv [n_loc, H_kv, d], dk_self, dv_self.

    ``groups`` restricts the computation to some KV heads (the other heads stay 0)."""
    nq, hq, d = q.shape
    hk = k_self.shape[1]
    grp = hq // hk
    if scale is None:
        scale = default_scale(d)
    off = chunk_offsets(chunk_len)
    dq = np.zeros((nq, hq, d))
    dk = np.zeros(k_loc.shape)
    dv = np.zeros(v_loc.shape)
    dks = np.zeros(k_self.shape)
    dvs = np.zeros(v_self.shape)
    for b in range(len(anchor)):
        lo, hi = visible_context(anchor, ctx_begin, b)
        local = []
        for c in range(len(chunk_start)):
            pos = int(chunk_start[c]) + np.arange(int(chunk_len[c]))
            local.append(off[c] + np.nonzero((pos >= lo) & (pos < hi))[0])
        local = np.concatenate(local) if local else np.zeros(0, np.int64)
        sl = slice(b * block_size, (b + 1) * block_size)
        for g in (range(hk) if groups is None else groups):
            hs = slice(g * grp, (g + 1) * grp)
            qr = _f64(q[sl, hs]).reshape(-1, d)
            dor = _f64(d_o[sl, hs]).reshape(-1, d)
            orow = _f64(o[sl, hs]).reshape(-1, d)
            lr = _f64(lse[sl, hs]).reshape(-1)
            keys = [_f64(k_loc[local, g])]
            vals = [_f64(v_loc[local, g])]
            if with_self:
                keys.append(_f64(k_self[sl, g]))
                vals.append(_f64(v_self[sl, g]))
            keys = np.concatenate(keys, 0)
            vals = np.concatenate(vals, 0)
            if keys.shape[0] == 0:
                continue
            s = scale * (qr @ keys.T)
            p = np.exp(s - lr[:, None])
            dd = (dor * orow).sum(axis=1)
            dp = dor @ vals.T
            ds = p * (dp - dd[:, None])
            dq[sl, hs] += (scale * (ds @ keys)).reshape(block_size, grp, d)
            dkeys = scale * (ds.T @ qr)
            dvals = p.T @ dor
            n_ctx = local.shape[0]
            np.add.at(dk[:, g], local, dkeys[:n_ctx])
            np.add.at(dv[:, g], local, dvals[:n_ctx])
            if with_self:
                dks[sl, g] += dkeys[n_ctx:]
                dvs[sl, g] += dvals[n_ctx:]
    return dq, dk, dv, dks, dvs
