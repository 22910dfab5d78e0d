"""Runs the fp64 oracle over (block, KV head) rows in worker processes.

Full-size parity needs the oracle on every row of the large workloads, which takes
minutes in one process.  The rows are independent, so they are split over a pool of
freshly spawned interpreters (no state inherited from a process that holds the GPU).
Each worker regenerates the seeded inputs itself from the workload's name, and every
value still comes from ``oracle``; this module only distributes the calls.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
from typing import Optional, Sequence

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_STATE = {}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def _init(name: str, q_scale: float, local: Optional[Sequence[int]], slot_of, n_slots: int,
          with_self: bool, backward: bool):
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from workloads import get_config, make_workload
    wl = make_workload(get_config(name))
    if q_scale != 1.0:
        wl.q = wl.q * np.float32(q_scale)
    ids = range(wl.n_chunks) if local is None else local
    k, v = wl.kv_chunks(ids)
    _STATE.update(wl=wl, k=k, v=v, starts=wl.chunk_start[list(ids)],
                  lens=wl.chunk_len[list(ids)], slot_of=np.asarray(slot_of), n_slots=n_slots,
                  with_self=with_self)


def _partials(blocks):
    import oracle
    s = _STATE
    wl = s["wl"]
    o, lse = oracle.slot_partials(wl.q, s["k"], s["v"], wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, wl.cfg.block_size, s["starts"], s["lens"],
                                  s["slot_of"], s["n_slots"], with_self=s["with_self"],
                                  blocks=blocks)
    B = wl.cfg.block_size
    rows = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks])
    return rows, o[:, rows], lse[:, rows]


def _merged(blocks):
    """Unchunked attention of some blocks (every query head), for workloads whose chunks,
    back to back, are the whole context in position order."""
    import oracle
    s = _STATE
    wl = s["wl"]
    hk = wl.cfg.n_kv_heads
    B = wl.cfg.block_size
    grp = wl.cfg.n_q_heads // hk
    rows = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks])
    o = np.zeros((len(blocks), B, wl.cfg.n_q_heads, wl.cfg.head_dim))
    lse = np.zeros((len(blocks), B, wl.cfg.n_q_heads))
    for i, b in enumerate(blocks):
        for g in range(hk):
            ob, lb = oracle.attention_block(wl.q, s["k"], s["v"], wl.k_self, wl.v_self,
                                            wl.anchor, wl.ctx_begin, B, b, g)
            o[i, :, g * grp:(g + 1) * grp] = ob
            lse[i, :, g * grp:(g + 1) * grp] = lb
    return rows, o.reshape(len(rows), *o.shape[2:]), lse.reshape(len(rows), -1)


_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def _pool(n: int, init_args):
    """A spawn pool of n workers with one BLAS thread each (the variables are read when a
    worker imports numpy, so they are set in the environment the workers inherit)."""
    saved = {k: os.environ.get(k) for k in _THREAD_VARS}
    for k in _THREAD_VARS:
        os.environ[k] = "1"
    try:
        return mp.get_context("spawn").Pool(n, initializer=_init, initargs=init_args)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def _run(fn, name, blocks_per_task, n_blocks, init_args):
    tasks = [list(range(b, min(b + blocks_per_task, n_blocks)))
             for b in range(0, n_blocks, blocks_per_task)]
    with _pool(_workers(), (name, *init_args)) as pool:
        return list(pool.imap_unordered(fn, tasks))


def slot_partials_all(name: str, n_blocks: int, n_q: int, n_q_heads: int, head_dim: int,
                      local, slot_of, n_slots: int, with_self: bool, q_scale: float = 1.0):
    """Every slot partial of a named workload: (O [n_out, N_q, H_q, d], LSE [n_out, N_q, H_q])."""
    n_out = n_slots + (1 if with_self else 0)
    o = np.full((n_out, n_q, n_q_heads, head_dim), np.nan)
    lse = np.full((n_out, n_q, n_q_heads), np.nan)
    for rows, po, pl in _run(_partials, name, 2, n_blocks,
                             (q_scale, local, slot_of, n_slots, with_self, False)):
        o[:, rows] = po
        lse[:, rows] = pl
    return o, lse


def merged_all(name: str, n_blocks: int, n_q: int, n_q_heads: int, head_dim: int,
               with_self: bool = True):
    """Unchunked attention of every query of a named workload over all its chunks."""
    o = np.full((n_q, n_q_heads, head_dim), np.nan)
    lse = np.full((n_q, n_q_heads), np.nan)
    for rows, po, pl in _run(_merged, name, 2, n_blocks,
                             (1.0, None, None, 1, with_self, False)):
        o[rows] = po
        lse[rows] = pl
    return o, lse


def _backward(groups):
    """Oracle gradients of the KV heads ``groups`` (their query heads, keys and draft keys),
    from the oracle's own unchunked forward (O, LSE)."""
    import oracle
    s = _STATE
    wl = s["wl"]
    c = wl.cfg
    out = []
    for g in groups:
        o, lse = oracle.attention(wl.q, s["k"], s["v"], wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, c.block_size, groups=[g])
        r = oracle.attention_backward(wl.q, s["k"], s["v"], wl.k_self, wl.v_self, wl.anchor,
                                      wl.ctx_begin, c.block_size, s["starts"], s["lens"],
                                      wl.d_o, np.nan_to_num(o), np.nan_to_num(lse, nan=0.0),
                                      groups=[g])
        grp = c.n_q_heads // c.n_kv_heads
        hs = slice(g * grp, (g + 1) * grp)
        out.append((g, r[0][:, hs], r[1][:, g], r[2][:, g], r[3][:, g], r[4][:, g]))
    return out


def backward_all(name: str):
    """Oracle gradients (dq, dk, dv, dk_self, dv_self) of every head of a named workload whose
    chunks, back to back, are the whole context in position order."""
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from workloads import get_config, make_workload
    wl = make_workload(get_config(name))
    c = wl.cfg
    n_loc = int(wl.chunk_len.sum())
    grp = c.n_q_heads // c.n_kv_heads
    dq = np.zeros(wl.q.shape)
    dk = np.zeros((n_loc, c.n_kv_heads, c.head_dim))
    dv = np.zeros_like(dk)
    dks = np.zeros(wl.k_self.shape)
    dvs = np.zeros_like(dks)
    tasks = [[g] for g in range(c.n_kv_heads)]
    with _pool(min(_workers(), len(tasks)), (name, 1.0, None, None, 1, True, True)) as pool:
        for res in pool.imap_unordered(_backward, tasks):
            for g, a, b_, c_, d_, e_ in res:
                dq[:, g * grp:(g + 1) * grp] = a
                dk[:, g], dv[:, g], dks[:, g], dvs[:, g] = b_, c_, d_, e_
    return dq, dk, dv, dks, dvs
