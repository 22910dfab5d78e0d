"""Shared helpers for the GPU parity tests: device upload of seeded workloads, the oracle's
own plan, and element-wise comparisons (expected values always come from ``oracle``)."""
from __future__ import annotations

import json
import math
import os
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


# Relative gates on O, per partial set, on top of the absolute ones above.  At sigma = 0.5
# attention is near-uniform over thousands of keys, so |O| is ~1e-2 and the absolute 2e-2
# bound alone would pass a dropped V tile; bf16 operands (P and V rounded to 8 significant
# bits, f32 accumulation) give relative errors near 2^-9 / sqrt(keys) per element, far
# inside these bounds.
REL_MAX_O = 2e-2        # max |dO| <= REL_MAX_O * max |O_ref|
REL_L2_O = 1e-2         # ||dO||_2 <= REL_L2_O * ||O_ref||_2

_STATS_PATH = os.environ.get("BSX_PARITY_STATS")


def record(what: str, **stats) -> None:
    """Appends one comparison's observed errors to the file named by BSX_PARITY_STATS."""
    if _STATS_PATH:
        with open(_STATS_PATH, "a") as f:
            f.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0],
                                "what": what, **stats}) + "\n")


def compare_partials(o_gpu, lse_gpu, o_ref, lse_ref, tol_o, tol_lse, what=""):
    """Element-wise check over the rows the oracle computed (non-NaN LSE).

    Empty rows (LSE = -inf) must be -inf on both sides; O is compared on finite rows only,
    where it must be finite.  Arrays of partials ([n_out, N_q, H_q, d]) are also gated per
    partial set (slot) by the relative bounds; merged outputs ([N_q, H_q, d]) as one set."""
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
    # relative gates per partial set
    sets = range(o_ref.shape[0]) if o_ref.ndim == 4 else [None]
    worst_rel, worst_l2 = 0.0, 0.0
    for si in sets:
        f = fin if si is None else fin[si]
        if not f.any():
            continue
        ref = o_ref[f] if si is None else o_ref[si][f]
        got = o_gpu[f] if si is None else o_gpu[si][f]
        err = got - ref
        ref_max = np.abs(ref).max()
        ref_l2 = np.linalg.norm(ref)
        rel = float(np.abs(err).max() / ref_max) if ref_max > 0 else 0.0
        l2 = float(np.linalg.norm(err) / ref_l2) if ref_l2 > 0 else 0.0
        assert ref_max > 0 or np.abs(err).max() == 0, f"{what} set {si}: O_ref is zero"
        assert rel <= REL_MAX_O, f"{what} set {si}: max|dO| / max|O| = {rel} > {REL_MAX_O}"
        assert l2 <= REL_L2_O, f"{what} set {si}: rel-L2(O) = {l2} > {REL_L2_O}"
        worst_rel, worst_l2 = max(worst_rel, rel), max(worst_l2, l2)
    stats.update(o_rel_set=worst_rel, o_l2_set=worst_l2)
    log(f"  {what}: rows={stats['n']} max|dLSE|={stats['lse']:.3g} max|dO|={stats['o']:.3g} "
        f"max|dO|/max|O| per set<={worst_rel:.3g} rel-L2 per set<={worst_l2:.3g}")
    record(what, **stats)
    assert stats["lse"] <= tol_lse, f"{what}: LSE error {stats['lse']} > {tol_lse}"
    assert stats["o"] <= tol_o, f"{what}: O error {stats['o']} > {tol_o}"
    return stats


# ---- launches with poisoned outputs and workspaces: every output is NaN and every
# workspace byte 0xFF before the call, so a row or buffer the library fails to write
# shows up as NaN (or as a garbage index) instead of passing on stale zeros

def nan_tensor(shape, dev="cuda"):
    return torch.full(tuple(shape), float("nan"), dtype=torch.float32, device=dev)


def poisoned_ws(nbytes: int, dev="cuda"):
    return torch.full((max(int(nbytes), 256),), 0xFF, dtype=torch.uint8, device=dev)


def run_fwd(shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks):
    n_out = chunks.n_slots + (1 if k_self is not None else 0)
    nq, hq, d = shape.n_queries, shape.n_q_heads, shape.head_dim
    o = nan_tensor((n_out, nq, hq, d), q.device)
    lse = nan_tensor((n_out, nq, hq), q.device)
    ws = poisoned_ws(bsx.fwd_workspace_bytes(shape, chunks), q.device)
    return bsx.attn_fwd(shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks, o, lse, ws)


def run_merge(o_parts, lse_parts, out_dtype: str = "f32"):
    rows = tuple(lse_parts.shape[1:])
    d = int(o_parts.shape[-1])
    o = torch.full((*rows, d), float("nan"), device=o_parts.device,
                   dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32)
    lse = nan_tensor(rows, o_parts.device)
    return bsx.lse_merge(o_parts, lse_parts, o, lse)


def run_bwd(shape, q, k, v, k_self, v_self, o, lse, d_o, anchor, ctx_begin, chunks):
    nq, hq, hk, d = shape.n_queries, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    nl = chunks.n_local
    dev = q.device
    out = (nan_tensor((nq, hq, d), dev), nan_tensor((nl, hk, d), dev),
           nan_tensor((nl, hk, d), dev),
           nan_tensor((nq, hk, d), dev) if k_self is not None else None,
           nan_tensor((nq, hk, d), dev) if k_self is not None else None)
    ws = poisoned_ws(bsx.bwd_workspace_bytes(shape, chunks), dev)
    return bsx.attn_bwd(shape, q, k, v, k_self, v_self, o, lse, d_o, anchor, ctx_begin, chunks,
                        out=out, ws=ws)


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
