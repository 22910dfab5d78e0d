"""Masked softmax attention, its per-slot partials.  (Oracle: test infrastructure only.)

Definition (Flash-dLLM page, "Method 1: I/O-Aware Fused KV-Cache Kernel", the
attention formula): O = softmax(Q K^T / sqrt(d)) V, taken row by row over the
keys a query may see (the mask rule of ``oracle.mask``).

Readings where the pages are silent:

* scale: 1/sqrt(d) unless the caller passes another one;
* grouped-query heads: query head ``h`` reads KV head ``h // (H_q / H_kv)``
  (contiguous groups; the Split-KV page's target-model table gives only the head
  counts);
* a partial over a key set T is the pair (O_T, LSE_T) with natural-log
  LSE_T = log sum_{k in T} exp(s_k) and O_T normalized within T,
  O_T = sum_{k in T} exp(s_k - LSE_T) v_k.  An empty T gives (O = 0, LSE = -inf);
* slot partials (Split-KV page, Abstract: key/value shards stay local, only
  query-sized tensors move): the context is cut into chunks, chunks are mapped to
  output slots, and a slot's partial is taken over the union of its chunks' keys
  that the query may see.  The draft block's own keys form one extra slot, last.
  The local K/V buffer holds the chunks concatenated in chunk index order.
"""
from __future__ import annotations

import math

import numpy as np

from .mask import visible_context


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def partial_attention(q_rows, keys, values, scale: float):
    """One partial: rows ``q_rows [n, d]`` over key set ``keys/values [m, d]``.

    Returns (O [n, d], LSE [n]); m == 0 gives (0, -inf)."""
    q_rows, keys, values = _f64(q_rows), _f64(keys), _f64(values)
    n, dv = q_rows.shape[0], values.shape[1]
    if keys.shape[0] == 0:
        return np.zeros((n, dv)), np.full(n, -np.inf)
    s = scale * (q_rows @ keys.T)
    m = s.max(axis=1)
    lse = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    w = np.exp(s - lse[:, None])
    return w @ values, lse


def _rows(x, b: int, block_size: int, heads):
    """Rows of block b for the given heads, ordered (query, head): [B*len(heads), d]."""
    blk = _f64(x[b * block_size:(b + 1) * block_size][:, heads])
    return blk.reshape(-1, blk.shape[-1])


def attention_block(q, k_ctx, v_ctx, k_self, v_self, anchor, ctx_begin, block_size: int,
                    b: int, g: int, scale: float = None):
    """Unchunked attention of block ``b``'s queries for the query heads of KV head ``g``.

    ``k_ctx/v_ctx`` hold the whole context at packed positions ``[0, S)``.
    Returns O [B, G, d] and LSE [B, G]."""
    hq, hk = q.shape[1], k_ctx.shape[1]
    grp = hq // hk
    if scale is None:
        scale = default_scale(q.shape[2])
    heads = list(range(g * grp, (g + 1) * grp))
    lo, hi = visible_context(anchor, ctx_begin, b)
    sl = slice(b * block_size, (b + 1) * block_size)
    keys = np.concatenate([_f64(k_ctx[lo:hi, g]), _f64(k_self[sl, g])], axis=0)
    vals = np.concatenate([_f64(v_ctx[lo:hi, g]), _f64(v_self[sl, g])], axis=0)
    o, lse = partial_attention(_rows(q, b, block_size, heads), keys, vals, scale)
    return o.reshape(block_size, grp, -1), lse.reshape(block_size, grp)


def attention(q, k_ctx, v_ctx, k_self, v_self, anchor, ctx_begin, block_size: int,
              scale: float = None, groups=None):
    """Unchunked masked attention for every query: O [N_q, H_q, d], LSE [N_q, H_q].

    ``groups`` restricts the computation to some KV heads (other heads stay NaN)."""
    nq, hq, d = q.shape
    hk = k_ctx.shape[1]
    grp = hq // hk
    o = np.full((nq, hq, v_ctx.shape[2]), np.nan)
    lse = np.full((nq, hq), np.nan)
    for b in range(len(anchor)):
        for g in (range(hk) if groups is None else groups):
            ob, lb = attention_block(q, k_ctx, v_ctx, k_self, v_self, anchor, ctx_begin,
                                     block_size, b, g, scale)
            o[b * block_size:(b + 1) * block_size, g * grp:(g + 1) * grp] = ob
            lse[b * block_size:(b + 1) * block_size, g * grp:(g + 1) * grp] = lb
    return o, lse


def chunk_offsets(chunk_len):
    """Local offset of each chunk in a buffer holding the chunks back to back in index order."""
    off, acc = [], 0
    for n in chunk_len:
        off.append(acc)
        acc += int(n)
    return off


def slot_keys(k_loc, v_loc, chunk_start, chunk_len, slot_of, s: int, lo: int, hi: int, g: int):
    """Keys/values of slot ``s`` (head ``g``) whose packed position lies in ``[lo, hi)``.

    Walks the slot's chunks in index order and, inside a chunk, its keys in position order."""
    off = chunk_offsets(chunk_len)
    ks, vs = [], []
    for c in range(len(chunk_start)):
        if int(slot_of[c]) != s:
            continue
        pos = int(chunk_start[c]) + np.arange(int(chunk_len[c]))
        local = off[c] + np.nonzero((pos >= lo) & (pos < hi))[0]
        ks.append(_f64(k_loc[local, g]))
        vs.append(_f64(v_loc[local, g]))
    if not ks:
        return np.zeros((0, k_loc.shape[2])), np.zeros((0, v_loc.shape[2]))
    return np.concatenate(ks, 0), np.concatenate(vs, 0)


def slot_partial_block(q, k_loc, v_loc, k_self, v_self, anchor, ctx_begin, block_size: int,
                       chunk_start, chunk_len, slot_of, n_slots: int, s: int, b: int, g: int,
                       scale: float = None):
    """Partial (O [B, G, d], LSE [B, G]) of slot ``s`` for block ``b``, KV head ``g``.

    ``s == n_slots`` is the draft block's own keys (the self slot)."""
    hq, hk = q.shape[1], k_self.shape[1]
    grp = hq // hk
    if scale is None:
        scale = default_scale(q.shape[2])
    heads = list(range(g * grp, (g + 1) * grp))
    if s == n_slots:
        sl = slice(b * block_size, (b + 1) * block_size)
        keys, vals = _f64(k_self[sl, g]), _f64(v_self[sl, g])
    else:
        lo, hi = visible_context(anchor, ctx_begin, b)
        keys, vals = slot_keys(k_loc, v_loc, chunk_start, chunk_len, slot_of, s, lo, hi, g)
    o, lse = partial_attention(_rows(q, b, block_size, heads), keys, vals, scale)
    return o.reshape(block_size, grp, -1), lse.reshape(block_size, grp)


def slot_partials(q, k_loc, v_loc, k_self, v_self, anchor, ctx_begin, block_size: int,
                  chunk_start, chunk_len, slot_of, n_slots: int, with_self: bool = True,
                  scale: float = None, blocks=None, groups=None):
    """All slot partials: O [n_slots(+1), N_q, H_q, d], LSE [n_slots(+1), N_q, H_q].

    ``blocks``/``groups`` restrict which rows are computed (others stay NaN)."""
    nq, hq, d = q.shape
    hk = k_self.shape[1]
    grp = hq // hk
    ns = n_slots + (1 if with_self else 0)
    o = np.full((ns, nq, hq, v_self.shape[2]), np.nan)
    lse = np.full((ns, nq, hq), np.nan)
    for s in range(ns):
        for b in (range(len(anchor)) if blocks is None else blocks):
            for g in (range(hk) if groups is None else groups):
                ob, lb = slot_partial_block(q, k_loc, v_loc, k_self, v_self, anchor, ctx_begin,
                                            block_size, chunk_start, chunk_len, slot_of,
                                            n_slots, s, b, g, scale)
                o[s, b * block_size:(b + 1) * block_size, g * grp:(g + 1) * grp] = ob
                lse[s, b * block_size:(b + 1) * block_size, g * grp:(g + 1) * grp] = lb
    return o, lse
