"""Shared helpers for the GPU parity tests: device upload of seeded workloads, the oracle's
own plan, and element-wise comparisons (expected values always come from ``oracle``)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import block_sparse_cross_amd as bsx

F32_TOL = 1e-5          # O and LSE, f32 inputs
BF16_TOL_O = 2e-2       # O, bf16 inputs with f32 accumulation
BF16_TOL_LSE = 2e-3     # LSE, bf16 inputs


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def shape_of(wl) -> bsx.Shape:
    c = wl.cfg
    return bsx.Shape(n_blocks=wl.n_blocks, block_size=c.block_size, n_q_heads=c.n_q_heads,
                     n_kv_heads=c.n_kv_heads, ctx_len=c.ctx_len, head_dim=c.head_dim,
                     dtype=c.dtype)


def to_dev(x: np.ndarray, dtype: str, dev="cuda"):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).to(dev)


def upload(wl, k_loc, v_loc, dev="cuda"):
    dt = wl.cfg.dtype
    out = dict(q=to_dev(wl.q, dt, dev), k=to_dev(k_loc, dt, dev), v=to_dev(v_loc, dt, dev),
               k_self=to_dev(wl.k_self, dt, dev), v_self=to_dev(wl.v_self, dt, dev),
               anchor=torch.from_numpy(wl.anchor).to(dev),
               ctx_begin=torch.from_numpy(wl.ctx_begin).to(dev))
    if wl.d_o is not None:
        out["d_o"] = to_dev(wl.d_o, dt, dev)
    return out


def oracle_plan(wl):
    """The oracle's own chunk costs, LPT result and local chunk selection."""
    c = wl.cfg
    counts, cost = oracle.chunk_costs(wl.anchor, wl.ctx_begin, c.block_size, wl.chunk_start,
                                      wl.chunk_len)
    n = wl.n_chunks
    if c.slot_mode == "per_chunk":
        return dict(counts=counts, cost=cost, slot_of=np.arange(n), n_slots=n,
                    local=np.arange(n), bin_of=None)
    bin_of, loads, ms, imb = oracle.lpt(cost, c.n_bins)
    bin_of = np.asarray(bin_of)
    if c.slot_mode == "lpt":
        return dict(counts=counts, cost=cost, slot_of=bin_of, n_slots=c.n_bins,
                    local=np.arange(n), bin_of=bin_of, loads=loads, makespan=ms, imbalance=imb)
    rank = max(range(c.n_bins), key=lambda j: (loads[j], -j))
    mine = np.nonzero(bin_of == rank)[0]
    return dict(counts=counts, cost=cost, slot_of=np.zeros(len(mine), np.int64), n_slots=1,
                local=mine, bin_of=bin_of, loads=loads, makespan=ms, imbalance=imb, rank=rank)


def compare_partials(o_gpu, lse_gpu, o_ref, lse_ref, tol_o, tol_lse, what=""):
    """Element-wise check over the rows the oracle computed (non-NaN LSE).

    Empty rows (LSE = -inf) must be -inf on both sides; O is compared on finite rows only."""
    lse_gpu = np.asarray(lse_gpu, np.float64)
    o_gpu = np.asarray(o_gpu, np.float64)
    sel = ~np.isnan(lse_ref)
    ref_empty = np.isneginf(lse_ref) & sel
    gpu_empty = np.isneginf(lse_gpu) & sel
    assert np.array_equal(ref_empty, gpu_empty), \
        f"{what}: empty-row sets differ ({ref_empty.sum()} vs {gpu_empty.sum()})"
    fin = sel & ~ref_empty
    if not fin.any():
        return dict(n=0, lse=0.0, o=0.0)
    dl = np.abs(lse_gpu[fin] - lse_ref[fin])
    do = np.abs(o_gpu[fin] - o_ref[fin])
    assert np.all(np.isfinite(dl)) and np.all(np.isfinite(do)), f"{what}: non-finite values"
    stats = dict(n=int(fin.sum()), lse=float(dl.max()), o=float(do.max()),
                 o_rel=float(do.max() / max(np.abs(o_ref[fin]).max(), 1e-30)))
    log(f"  {what}: rows={stats['n']} max|dLSE|={stats['lse']:.3g} max|dO|={stats['o']:.3g} "
        f"max|dO|/max|O|={stats['o_rel']:.3g}")
    assert stats["lse"] <= tol_lse, f"{what}: LSE error {stats['lse']} > {tol_lse}"
    assert stats["o"] <= tol_o, f"{what}: O error {stats['o']} > {tol_o}"
    return stats


def sample_pairs(wl, n: int, seed: int):
    """(block, kv head) pairs: first and last block plus random ones."""
    rng = np.random.default_rng(seed)
    nb, hk = wl.n_blocks, wl.cfg.n_kv_heads
    pairs = {(0, 0), (nb - 1, hk - 1)}
    while len(pairs) < min(n, nb * hk):
        pairs.add((int(rng.integers(nb)), int(rng.integers(hk))))
    return sorted(pairs)


def tolerances(dtype: str):
    return (F32_TOL, F32_TOL) if dtype == "f32" else (BF16_TOL_O, BF16_TOL_LSE)


def useful_flops(anchor, ctx_begin, block_size, n_q_heads, head_dim, self_keys=True):
    """4 * d * H_q * sum over queries of visible keys (context + own block)."""
    vis = (np.asarray(anchor) - np.asarray(ctx_begin)).sum() * block_size
    if self_keys:
        vis += len(anchor) * block_size * block_size
    return 4.0 * head_dim * n_q_heads * float(vis)


__all__ = ["math"]
