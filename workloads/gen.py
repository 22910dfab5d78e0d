"""Seeded input generation.

Everything here is input synthesis: random draws, dtype rounding of the draws,
and the packing of variable-length samples into one context.  No visibility,
cost, plan or attention arithmetic lives here.

Draw recipe (one ``numpy.random.default_rng(seed)`` stream, in this order):
  1. packed workloads only: ``n_samples`` lengths ``round(exp(U[ln len_lo, ln len_hi]))``,
     all redrawn together while their sum exceeds ``ctx_len``; the remaining tail of the
     context is a padding segment that holds no anchors;
  2. anchors: per sample, drawn uniformly without replacement (single-sample workloads from
     ``[anchor_lo, anchor_hi)``, packed workloads from ``[0, L_i)`` with ``L_i // anchor_every``
     anchors), sorted ascending, shifted to packed (global) positions;
  3. ``Q [N_q, H_q, d]``, ``K_self [N_q, H_kv, d]``, ``V_self [N_q, H_kv, d]``, then
     ``dO [N_q, H_q, d]`` for training workloads, each ``standard_normal(float32) * sigma``
     (``dO`` with sigma 1).
Context keys/values are drawn per chunk from ``default_rng([seed, 1, c])`` (K chunk then V
chunk), so one rank's local chunks can be drawn without the rest.  Standalone merge sets are
drawn per set from ``default_rng([seed, 2, p])`` (O then LSE).  bf16 workloads round every
floating draw to bfloat16 with round-to-nearest-even and keep the rounded values.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from .configs import WorkloadConfig


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are exactly bfloat16 (as uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclass
class Workload:
    cfg: WorkloadConfig
    sample_len: List[int]            # lengths of the packed samples (single sample: [S])
    sample_start: List[int]          # packed offset of each sample
    anchor: np.ndarray               # int64 [n_blocks]: packed anchor position of each block
    ctx_begin: np.ndarray            # int64 [n_blocks]: packed start of the block's sample
    chunk_start: np.ndarray          # int64 [n_chunks]: packed start of each KV chunk
    chunk_len: np.ndarray            # int64 [n_chunks]
    q: np.ndarray                    # float32 [N_q, H_q, d]
    k_self: np.ndarray               # float32 [N_q, H_kv, d]
    v_self: np.ndarray               # float32 [N_q, H_kv, d]
    d_o: Optional[np.ndarray] = None  # float32 [N_q, H_q, d] (training workloads)
    extra: dict = field(default_factory=dict)

    @property
    def n_blocks(self) -> int:
        return int(self.anchor.shape[0])

    @property
    def n_queries(self) -> int:
        return self.n_blocks * self.cfg.block_size

    @property
    def n_chunks(self) -> int:
        return int(self.chunk_start.shape[0])

    def kv_chunks(self, chunk_ids: Optional[Sequence[int]] = None):
        """Context K and V for the given chunks, concatenated in the given order."""
        if chunk_ids is None:
            chunk_ids = range(self.n_chunks)
        return draw_kv_chunks(self.cfg, [int(self.chunk_len[c]) for c in chunk_ids],
                              list(chunk_ids))


def _round(cfg: WorkloadConfig, x: np.ndarray) -> np.ndarray:
    return round_to_bf16(x) if cfg.dtype == "bf16" else x.astype(np.float32)


def draw_kv_chunks(cfg: WorkloadConfig, lens: Sequence[int], chunk_ids: Sequence[int]):
    hk, d = cfg.n_kv_heads, cfg.head_dim
    ks, vs = [], []
    for c, n in zip(chunk_ids, lens):
        rng = np.random.default_rng([cfg.seed, 1, int(c)])
        ks.append(_round(cfg, rng.standard_normal((n, hk, d), dtype=np.float32) * cfg.sigma))
        vs.append(_round(cfg, rng.standard_normal((n, hk, d), dtype=np.float32) * cfg.sigma))
    if not ks:
        z = np.zeros((0, hk, d), np.float32)
        return z, z.copy()
    return np.concatenate(ks, 0), np.concatenate(vs, 0)


def draw_merge_sets(cfg: WorkloadConfig, n_sets: int, n_rows: int, head_dim: int,
                    sets: Optional[Sequence[int]] = None, rows: Optional[np.ndarray] = None):
    """Seeded partial (O, LSE) sets: O ~ N(0,1) fp32 [n_rows, d], LSE ~ N(0,1) + shift.

    ``rows`` selects a subset of rows (the full set is drawn, then indexed)."""
    if sets is None:
        sets = range(n_sets)
    os_, ls_ = [], []
    for p in sets:
        rng = np.random.default_rng([cfg.seed, 2, int(p)])
        o = rng.standard_normal((n_rows, head_dim), dtype=np.float32)
        lse = rng.standard_normal(n_rows, dtype=np.float32) + np.float32(cfg.merge_lse_shift)
        if rows is not None:
            o, lse = o[rows], lse[rows]
        os_.append(o)
        ls_.append(lse)
    return np.stack(os_, 0), np.stack(ls_, 0)


def _draw_lengths(cfg: WorkloadConfig, rng: np.random.Generator) -> List[int]:
    lo, hi = np.log(cfg.len_lo), np.log(cfg.len_hi)
    while True:
        lens = [int(np.rint(np.exp(rng.uniform(lo, hi)))) for _ in range(cfg.n_samples)]
        if sum(lens) <= cfg.ctx_len:
            return lens


def make_workload(cfg: WorkloadConfig, seed: Optional[int] = None) -> Workload:
    if seed is not None and seed != cfg.seed:
        from dataclasses import replace
        cfg = replace(cfg, seed=seed)
    rng = np.random.default_rng(cfg.seed)
    if cfg.packed:
        lens = _draw_lengths(cfg, rng)
    else:
        lens = [cfg.ctx_len]
    starts = [int(s) for s in np.concatenate([[0], np.cumsum(lens)[:-1]])]

    anchors, begins = [], []
    for s0, n in zip(starts, lens):
        if cfg.packed:
            k, lo, hi = n // cfg.anchor_every, 0, n
        else:
            k, lo, hi = cfg.n_anchors, cfg.anchor_lo, cfg.anchor_hi
        a = np.sort(rng.choice(hi - lo, size=k, replace=False).astype(np.int64) + lo)
        anchors.append(a + s0)
        begins.append(np.full(k, s0, np.int64))
    anchor = np.concatenate(anchors).astype(np.int64)
    ctx_begin = np.concatenate(begins).astype(np.int64)

    nq = anchor.shape[0] * cfg.block_size
    hq, hk, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = _round(cfg, rng.standard_normal((nq, hq, d), dtype=np.float32) * cfg.sigma)
    k_self = _round(cfg, rng.standard_normal((nq, hk, d), dtype=np.float32) * cfg.sigma)
    v_self = _round(cfg, rng.standard_normal((nq, hk, d), dtype=np.float32) * cfg.sigma)
    d_o = None
    if cfg.backward:
        d_o = _round(cfg, rng.standard_normal((nq, hq, d), dtype=np.float32))

    nc = cfg.n_chunks
    chunk_start = np.arange(nc, dtype=np.int64) * cfg.chunk_len
    chunk_len = np.full(nc, cfg.chunk_len, np.int64)
    return Workload(cfg=cfg, sample_len=lens, sample_start=starts, anchor=anchor,
                    ctx_begin=ctx_begin, chunk_start=chunk_start, chunk_len=chunk_len,
                    q=q, k_self=k_self, v_self=v_self, d_o=d_o)


def custom_workload(*, seed: int, ctx_len: int, n_q_heads: int, n_kv_heads: int,
                    head_dim: int = 128, dtype: str = "bf16", sigma: float = 0.5,
                    block_size: int = 16, anchor: Sequence[int], ctx_begin: Sequence[int],
                    chunk_start: Sequence[int], chunk_len: Sequence[int],
                    backward: bool = False) -> Workload:
    """A workload with explicitly given anchors and chunking (edge cases, ragged tails).

    Q, K_self, V_self (and dO) are drawn as in ``make_workload`` step 3; context K/V are drawn
    per chunk by ``Workload.kv_chunks``."""
    from .configs import WorkloadConfig
    cfg = WorkloadConfig(name="custom", seed=seed, ctx_len=ctx_len, n_q_heads=n_q_heads,
                         n_kv_heads=n_kv_heads, head_dim=head_dim, dtype=dtype, sigma=sigma,
                         block_size=block_size, chunk_len=max(1, int(max(chunk_len, default=1))),
                         backward=backward)
    rng = np.random.default_rng(seed)
    anchor = np.asarray(anchor, np.int64)
    nq = anchor.shape[0] * block_size
    q = _round(cfg, rng.standard_normal((nq, n_q_heads, head_dim), dtype=np.float32) * sigma)
    k_self = _round(cfg, rng.standard_normal((nq, n_kv_heads, head_dim), dtype=np.float32) * sigma)
    v_self = _round(cfg, rng.standard_normal((nq, n_kv_heads, head_dim), dtype=np.float32) * sigma)
    d_o = None
    if backward:
        d_o = _round(cfg, rng.standard_normal((nq, n_q_heads, head_dim), dtype=np.float32))
    return Workload(cfg=cfg, sample_len=[ctx_len], sample_start=[0], anchor=anchor,
                    ctx_begin=np.asarray(ctx_begin, np.int64),
                    chunk_start=np.asarray(chunk_start, np.int64),
                    chunk_len=np.asarray(chunk_len, np.int64), q=q, k_self=k_self,
                    v_self=v_self, d_o=d_o)
