"""GPU parity on seeded random configurations against the fp64 oracle: query-head groups,
block sizes, context lengths, chunk layouts (gaps, unsorted lists, overlapping and
zero-length chunks), slot maps with empty slots, anchors at the edges of the context, with
and without the draft blocks' own keys.  Each configuration runs the forward partials, the
merge and the backward through the C ABI and is compared in full; the sizes keep the
oracle at a second or two per case.  The draw itself is checked on the CPU."""
from dataclasses import dataclass
from typing import List

import numpy as np
import pytest
import torch

import block_sparse_cross_amd as bsx
import oracle
from parity_helpers import (compare_partials, log, record, run_bwd, run_fwd, run_merge,
                            shape_of, tolerances, upload)
from workloads.gen import custom_workload

GRAD_MAX_REL = 2e-2   # gradients: max abs error <= 2e-2 * max |reference|
GRAD_L2_REL = 1e-2    # and relative L2 error <= 1e-2 (bf16 operands, f32 accumulation)

N_BF16 = 120          # bf16 configurations (forward, merge, backward)
N_F32 = 40            # f32 configurations (forward and merge)


@dataclass
class Draw:
    seed: int
    dtype: str
    ctx_len: int
    n_q_heads: int
    n_kv_heads: int
    block_size: int
    anchor: List[int]
    ctx_begin: List[int]
    chunk_start: List[int]
    chunk_len: List[int]
    slot_of: List[int]
    n_slots: int
    with_self: bool


def draw(seed: int, dtype: str) -> Draw:
    """One valid configuration: 0 <= ctx_begin <= anchor <= S, chunks inside [0, S)."""
    rng = np.random.default_rng(10_000 + seed)
    hk = int(rng.choice([1, 2, 3, 4]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8]))
    while hk * G > 16:
        G -= 1
    B = int(rng.choice([1, 2, 3, 5, 7, 16, 17, 31, 32, 64, 80, 128, 256]))
    nb = int(rng.integers(1, 13 if B <= 32 else 5))
    S = int(rng.integers(1, 6000))
    mode = int(rng.integers(0, 3))
    if mode < 2:
        # a partition of [0, S) into runs, some dropped (gaps), in order or shuffled
        n = int(rng.integers(1, 13))
        cuts = np.unique(np.concatenate([[0, S], rng.integers(0, S + 1, size=n - 1)]))
        runs = [(int(a), int(b - a)) for a, b in zip(cuts[:-1], cuts[1:])]
        keep = [r for r in runs if rng.random() < 0.8] or runs[:1]
        if mode == 1:
            keep = [keep[i] for i in rng.permutation(len(keep))]
        cs, cl = [a for a, _ in keep], [n for _, n in keep]
    else:
        # independent intervals: overlapping, zero-length, unsorted
        n = int(rng.integers(1, 9))
        cs, cl = [], []
        for _ in range(n):
            a = int(rng.integers(0, S + 1))
            cs.append(a)
            cl.append(0 if rng.random() < 0.15 else int(rng.integers(0, S - a + 1)))
    n_slots = int(rng.integers(1, len(cs) + 2))  # the last slots may stay empty
    slot_of = [int(x) for x in rng.integers(0, n_slots, size=len(cs))]
    anchor, begin = [], []
    for _ in range(nb):
        u = rng.random()
        a = 0 if u < 0.1 else S if u < 0.25 else int(rng.integers(0, S + 1))
        b = 0 if rng.random() < 0.5 else int(rng.integers(0, a + 1))
        anchor.append(a)
        begin.append(b)
    return Draw(seed=seed, dtype=dtype, ctx_len=S, n_q_heads=hk * G, n_kv_heads=hk,
                block_size=B, anchor=anchor, ctx_begin=begin, chunk_start=cs, chunk_len=cl,
                slot_of=slot_of, n_slots=n_slots, with_self=bool(rng.random() < 0.75))


def _workload(d: Draw, backward: bool):
    return custom_workload(seed=20_000 + d.seed, ctx_len=d.ctx_len, n_q_heads=d.n_q_heads,
                           n_kv_heads=d.n_kv_heads, dtype=d.dtype,
                           sigma=1.0 if d.dtype == "f32" else 0.5, block_size=d.block_size,
                           anchor=d.anchor, ctx_begin=d.ctx_begin, chunk_start=d.chunk_start,
                           chunk_len=d.chunk_len, backward=backward)


@pytest.mark.parametrize("seed", range(N_BF16 + N_F32))
def test_draws_are_valid_and_small(seed):
    """Every draw satisfies the ABI's input rules and keeps the oracle's work small."""
    d = draw(seed, "bf16" if seed < N_BF16 else "f32")
    S = d.ctx_len
    assert d.n_q_heads % d.n_kv_heads == 0 and d.n_q_heads <= 16
    assert 1 <= d.block_size <= 256 and len(d.anchor) == len(d.ctx_begin) >= 1
    assert all(0 <= b <= a <= S for a, b in zip(d.anchor, d.ctx_begin))
    assert all(0 <= s and 0 <= n and s + n <= S for s, n in zip(d.chunk_start, d.chunk_len))
    assert len(d.slot_of) == len(d.chunk_start) >= 1
    assert all(0 <= s < d.n_slots for s in d.slot_of)
    rows = len(d.anchor) * d.block_size * d.n_q_heads
    assert rows * (sum(d.chunk_len) + d.block_size) <= 60_000_000


def _check_grad(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    log(f"  {name}: max|ref|={scale:.3g} max err={err:.3g} rel-L2={l2:.3g}")
    record(name, max_ref=float(scale), max_err=float(err), rel=float(err / max(scale, 1e-30)),
           l2=float(l2))
    if scale == 0:
        assert err == 0, f"{name}: {err} where the reference is zero"
        return
    assert err <= GRAD_MAX_REL * scale, f"{name}: max error {err} > {GRAD_MAX_REL} * {scale}"
    assert l2 <= GRAD_L2_REL, f"{name}: relative L2 error {l2} > {GRAD_L2_REL}"


def _describe(d: Draw) -> str:
    return (f"seed={d.seed} {d.dtype} S={d.ctx_len} H_q={d.n_q_heads} H_kv={d.n_kv_heads} "
            f"B={d.block_size} blocks={len(d.anchor)} chunks={len(d.chunk_start)} "
            f"slots={d.n_slots} self={d.with_self}")


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_BF16 + N_F32))
def test_random_config(seed):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dtype = "bf16" if seed < N_BF16 else "f32"
    d = draw(seed, dtype)
    backward = dtype == "bf16"
    log(f"random config: {_describe(d)}")
    wl = _workload(d, backward)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    ks = dev["k_self"] if d.with_self else None
    vs = dev["v_self"] if d.with_self else None
    cs, cl = np.asarray(d.chunk_start, np.int64), np.asarray(d.chunk_len, np.int64)
    B, hq = d.block_size, d.n_q_heads
    tol_o, tol_l = tolerances(dtype)

    # forward partials with the drawn slot map, every row
    o_part, lse_part = run_fwd(shape, dev["q"], dev["k"], dev["v"], ks, vs, dev["anchor"],
                               dev["ctx_begin"], bsx.Chunks(cs, cl, d.slot_of, d.n_slots))
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, B, cs, cl, np.asarray(d.slot_of), d.n_slots,
                                  with_self=d.with_self)
    compare_partials(o_part.cpu().numpy(), lse_part.cpu().numpy(), ro, rl, tol_o, tol_l,
                     "partials")

    # the merge of those partials against the oracle's merge of its own
    mo, ml = run_merge(o_part, lse_part)
    nq = wl.q.shape[0]
    uo, ul = oracle.lse_merge(ro.reshape(ro.shape[0], nq * hq, -1),
                              rl.reshape(rl.shape[0], nq * hq))
    uo, ul = uo.reshape(nq, hq, -1), ul.reshape(nq, hq)
    compare_partials(mo.cpu().numpy(), ml.cpu().numpy(), uo, ul, tol_o, tol_l, "merged")
    if not backward:
        return

    # the backward from the GPU's own merged forward; the oracle's from its own
    grads = run_bwd(shape, dev["q"], dev["k"], dev["v"], ks, vs, mo, ml, dev["d_o"],
                    dev["anchor"], dev["ctx_begin"], bsx.Chunks(cs, cl))
    torch.cuda.synchronize()
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, B, cs, cl, wl.d_o, np.nan_to_num(uo), ul,
                                  with_self=d.with_self)
    names = ["dq", "dk", "dv", "dk_self", "dv_self"]
    for name, got, ref in zip(names[:5 if d.with_self else 3], grads, r):
        _check_grad(name, got.cpu().numpy(), ref)
