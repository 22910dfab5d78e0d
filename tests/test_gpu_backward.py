"""GPU parity of the attention backward (bf16 inputs, f32 gradients) against the fp64 oracle.

The gradients of the training workload have no tolerance of their own, so each gradient
tensor must satisfy: max abs error <= 2e-2 * max |reference| and relative L2 error <= 1e-2
(bf16 operands with f32 accumulation; gradients are small because softmax weights are ~1/n).
The GPU path takes its merged forward (O, LSE) from its own forward + merge, as a training
step does; the oracle uses its own fp64 forward.
"""
import numpy as np
import pytest
import torch

import block_sparse_cross_amd as bsx
import oracle
import oracle_pool
from parity_helpers import log, record, run_bwd, run_fwd, run_merge, shape_of, upload
from workloads import get_config, make_workload
from workloads.gen import custom_workload

pytestmark = pytest.mark.gpu

MAX_REL = 2e-2
L2_REL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _check(name, got, ref, mask=None):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    log(f"  {name}: max|ref|={scale:.3g} max err={err:.3g} ({err / max(scale, 1e-30):.3g} rel) "
        f"rel-L2={l2:.3g}")
    record(name, max_ref=float(scale), max_err=float(err), rel=float(err / max(scale, 1e-30)),
           l2=float(l2))
    if scale == 0:
        assert err == 0, name
        return
    assert err <= MAX_REL * scale, f"{name}: max error {err} > {MAX_REL} * {scale}"
    assert l2 <= L2_REL, f"{name}: relative L2 error {l2} > {L2_REL}"


def _gpu_forward_backward(wl, k_loc, v_loc, chunks, with_self=True):
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    ks = dev["k_self"] if with_self else None
    vs = dev["v_self"] if with_self else None
    o_part, lse_part = run_fwd(shape, dev["q"], dev["k"], dev["v"], ks, vs, dev["anchor"],
                               dev["ctx_begin"], chunks)
    o, lse = run_merge(o_part, lse_part)
    grads = run_bwd(shape, dev["q"], dev["k"], dev["v"], ks, vs, o, lse, dev["d_o"],
                    dev["anchor"], dev["ctx_begin"], chunks)
    torch.cuda.synchronize()
    return [None if x is None else x.cpu().numpy() for x in grads]


CASES = {
    # name: (S, H_q, H_kv, B, anchors, begins, chunk starts, chunk lens)
    "gqa4_ragged": (3000, 8, 2, 16, [0, 5, 777, 1500, 2999, 3000], None,
                    [0, 1000, 1999, 2000], [1000, 999, 1, 1000]),
    "gqa8_packed": (4096, 32, 4, 16, [100, 1500, 1600, 4000, 2500], [0, 0, 1000, 2400, 2400],
                    list(range(0, 4096, 512)), [512] * 8),
    "mha_block5": (700, 4, 4, 5, [3, 100, 650, 699, 700, 0, 350], None, [0, 350], [350, 350]),
    "gqa2_block8": (900, 8, 4, 8, [899, 450, 10], None, [0, 300, 600], [300, 300, 300]),
    # chunks listed out of position order: the backward walks its list unsorted
    "unsorted_chunks": (3000, 8, 2, 16, [100, 2999, 1500, 600], None,
                        [2000, 0, 1000], [1000, 1000, 1000]),
    # 300 chunks (more than the 256-entry LDS copies): chunk list walked from memory
    "many_small_chunks": (4800, 8, 2, 16, [30, 4800, 2400, 1111, 4000], None,
                          list(range(0, 4800, 16)), [16] * 300),
    # draft blocks larger than a key tile: self keys of several 64-key tiles per block
    "block80_gqa4": (3000, 8, 2, 80, [0, 1500, 3000, 2999], None, [0, 1000, 2000],
                     [1000, 1000, 1000]),
    "block256_gqa2": (2048, 4, 2, 256, [700, 2048, 1], [0, 100, 0], [0, 1024], [1024, 1024]),
    # 64-key tiles spanning distant chunks; rows 64..127 (positions 2024..2087) are seen
    # by no block, so their dK/dV must be exactly zero
    "split_tiles_unseen": (3000, 8, 2, 16, [20, 2010], None, [0, 2000, 900], [40, 100, 30]),
    # query-head groups that do not divide the 32-row steps or 128-row tiles (a block's
    # rows end inside a step, a query's heads straddle tiles), odd block sizes
    "gqa3_block7": (1800, 6, 2, 7, [0, 5, 900, 1799, 1800, 333, 1200], None,
                    [0, 600, 1200], [600, 600, 600]),
    "gqa5_block13": (1000, 10, 2, 13, [1000, 1, 500, 999, 250], None,
                     [0, 250, 500, 750], [250, 250, 250, 250]),
    "gqa7_block33": (2100, 7, 1, 33, [2100, 64, 1000, 2099], [0, 0, 500, 1000],
                     [100, 1100], [1000, 1000]),
    # 2100 chunks of 2 keys: more entries than the dQ plan keeps in LDS
    "many_tiny_chunks": (4200, 4, 2, 4, [0, 4200, 2100, 1, 3333, 777], None,
                         list(range(0, 4200, 2)), [2] * 2100),
    # the same past the LDS copy, listed out of position order: the plan walks the whole
    # list from memory for every row tile
    "many_chunks_unsorted": (2400, 4, 2, 4, [0, 2400, 1200, 7, 2399], None,
                             [int(x) for x in np.random.default_rng(3).permutation(
                                 np.arange(0, 2400, 4))], [4] * 600),
    # 600 row tiles per KV head: more than the dQ plan keeps in LDS (the chunk list
    # still fits there)
    "plan_many_row_tiles": (512, 8, 2, 32,
                            [int(x) for x in np.random.default_rng(7).integers(0, 513, 600)],
                            None, [256, 0], [256, 256]),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_backward_small_full(case):
    S, hq, hk, B, an, be, cs, cl = CASES[case]
    log(f"backward, {case}")
    be = [0] * len(an) if be is None else be
    wl = custom_workload(seed=11, ctx_len=S, n_q_heads=hq, n_kv_heads=hk, block_size=B,
                         anchor=an, ctx_begin=be, chunk_start=cs, chunk_len=cl, backward=True)
    k_loc, v_loc = wl.kv_chunks()
    chunks = bsx.Chunks(cs, cl)
    dq, dk, dv, dks, dvs = _gpu_forward_backward(wl, k_loc, v_loc, chunks)
    # reference (O, LSE): every local chunk as one slot plus the draft keys, merged (the
    # chunks need not cover the context, so no global key array is built)
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, B, np.asarray(cs), np.asarray(cl),
                                  np.zeros(len(cs), np.int64), 1)
    nq = wl.q.shape[0]
    mo, ml = oracle.lse_merge(ro.reshape(2, nq * hq, -1), rl.reshape(2, nq * hq))
    o, lse = mo.reshape(nq, hq, -1), ml.reshape(nq, hq)
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, B, np.asarray(cs), np.asarray(cl), wl.d_o, o, lse)
    for name, got, ref in zip(["dq", "dk", "dv", "dk_self", "dv_self"], [dq, dk, dv, dks, dvs], r):
        _check(name, got, ref)


def test_backward_unseen_tile_is_zero():
    """The key tile no block sees (see the split_tiles_unseen case) comes out as exact zeros."""
    S, hq, hk, B, an, be, cs, cl = CASES["split_tiles_unseen"]
    wl = custom_workload(seed=13, ctx_len=S, n_q_heads=hq, n_kv_heads=hk, block_size=B,
                         anchor=an, ctx_begin=[0] * len(an), chunk_start=cs, chunk_len=cl,
                         backward=True)
    k_loc, v_loc = wl.kv_chunks()
    dq, dk, dv, dks, dvs = _gpu_forward_backward(wl, k_loc, v_loc, bsx.Chunks(cs, cl))
    assert np.all(dk[64:128] == 0) and np.all(dv[64:128] == 0)
    assert np.any(dk[:64] != 0) and np.any(dk[140:] != 0)


def test_backward_overlapping_chunks_without_self():
    """Two chunks share positions (their keys are distinct rows at the same positions): the
    chunk list is sorted but not disjoint.  One slot holds every chunk, no self keys."""
    cs, cl = [0, 700, 1500], [1000, 1000, 300]
    wl = custom_workload(seed=14, ctx_len=2048, n_q_heads=8, n_kv_heads=2, block_size=16,
                         anchor=[900, 2048, 1600, 50], ctx_begin=[0] * 4, chunk_start=cs,
                         chunk_len=cl, backward=True)
    k_loc, v_loc = wl.kv_chunks()
    chunks = bsx.Chunks(cs, cl, [0, 0, 0], 1)
    dq, dk, dv, dks, dvs = _gpu_forward_backward(wl, k_loc, v_loc, chunks, with_self=False)
    o_p, lse_p = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                      wl.ctx_begin, 16, np.asarray(cs), np.asarray(cl), [0, 0, 0],
                                      1, with_self=False)
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, np.asarray(cs), np.asarray(cl), wl.d_o,
                                  np.nan_to_num(o_p[0]), lse_p[0], with_self=False)
    for name, got, ref in zip(["dq", "dk", "dv"], [dq, dk, dv], r[:3]):
        _check(name, got, ref)


def test_backward_rank_share_without_self():
    """One rank's non-contiguous chunks, no self keys: local dK/dV exact, dQ is this share."""
    wl = custom_workload(seed=12, ctx_len=8192, n_q_heads=32, n_kv_heads=8, block_size=16,
                         anchor=[0, 900, 3000, 5000, 8192, 6100], ctx_begin=[0] * 6,
                         chunk_start=[4096, 1024, 7168], chunk_len=[1024, 1024, 1024],
                         backward=True)
    k_loc, v_loc = wl.kv_chunks()
    chunks = bsx.Chunks(wl.chunk_start, wl.chunk_len, [0, 0, 0], 1)
    dq, dk, dv, dks, dvs = _gpu_forward_backward(wl, k_loc, v_loc, chunks, with_self=False)
    assert dks is None and dvs is None
    # the GPU's (O, LSE) here are the rank-local partial: the oracle uses the same definition
    pos = np.concatenate([np.arange(s, s + c) for s, c in zip(wl.chunk_start, wl.chunk_len)])
    o_p, lse_p = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                      wl.ctx_begin, 16, wl.chunk_start, wl.chunk_len, [0, 0, 0],
                                      1, with_self=False)
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, wl.chunk_start, wl.chunk_len, wl.d_o,
                                  np.nan_to_num(o_p[0]), lse_p[0], with_self=False)
    for name, got, ref in zip(["dq", "dk", "dv"], [dq, dk, dv], r[:3]):
        _check(name, got, ref)
    assert pos.shape[0] == dk.shape[0]


def test_backward_training_workload_all_heads():
    """The full-size training step (8 packed samples, 131072 keys, 16 LPT bins); the oracle
    computes every gradient of every KV head (its query heads, keys and draft keys)."""
    wl = make_workload(get_config("train_pack128k"))
    c = wl.cfg
    log(f"backward, {c.name}: blocks={wl.n_blocks}, all heads")
    k_loc, v_loc = wl.kv_chunks()
    _, cost = oracle.chunk_costs(wl.anchor, wl.ctx_begin, c.block_size, wl.chunk_start,
                                 wl.chunk_len)
    bin_of, *_ = oracle.lpt(cost, c.n_bins)
    chunks = bsx.Chunks(wl.chunk_start, wl.chunk_len, bin_of, c.n_bins)
    dq, dk, dv, dks, dvs = _gpu_forward_backward(wl, k_loc, v_loc, chunks)
    r = oracle_pool.backward_all(c.name)
    _check("dq", dq, r[0])
    _check("dk", dk, r[1])
    _check("dv", dv, r[2])
    _check("dk_self", dks, r[3])
    _check("dv_self", dvs, r[4])
    # keys past the last sample (the padding tail) are seen by no query
    tail = sum(wl.sample_len)
    assert np.all(dk[tail:] == 0) and np.all(dv[tail:] == 0)


def test_backward_rank_share_sorted_chunks():
    """One rank's chunks listed in position order, no self keys; some blocks' ranges fall
    between the chunks (their rows see none of the local keys)."""
    wl = custom_workload(seed=15, ctx_len=8192, n_q_heads=32, n_kv_heads=8, block_size=16,
                         anchor=[0, 900, 3000, 5000, 8192, 6100, 2100], ctx_begin=[0] * 7,
                         chunk_start=[1024, 4096, 7168], chunk_len=[1024, 1024, 1024],
                         backward=True)
    k_loc, v_loc = wl.kv_chunks()
    chunks = bsx.Chunks(wl.chunk_start, wl.chunk_len, [0, 0, 0], 1)
    dq, dk, dv, dks, dvs = _gpu_forward_backward(wl, k_loc, v_loc, chunks, with_self=False)
    o_p, lse_p = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                      wl.ctx_begin, 16, wl.chunk_start, wl.chunk_len, [0, 0, 0],
                                      1, with_self=False)
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, wl.chunk_start, wl.chunk_len, wl.d_o,
                                  np.nan_to_num(o_p[0]), lse_p[0], with_self=False)
    for name, got, ref in zip(["dq", "dk", "dv"], [dq, dk, dv], r[:3]):
        _check(name, got, ref)


def test_backward_is_deterministic():
    wl = custom_workload(seed=13, ctx_len=2048, n_q_heads=16, n_kv_heads=4, block_size=16,
                         anchor=[700, 2048, 1500], ctx_begin=[0, 0, 0], chunk_start=[0, 1024],
                         chunk_len=[1024, 1024], backward=True)
    k_loc, v_loc = wl.kv_chunks()
    chunks = bsx.Chunks(wl.chunk_start, wl.chunk_len)
    a = _gpu_forward_backward(wl, k_loc, v_loc, chunks)
    b = _gpu_forward_backward(wl, k_loc, v_loc, chunks)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_custom_scale():
    """A softmax scale other than 1/sqrt(d) (0.3) in both passes: P, dS and the scale of dQ
    and dK all follow it (GQA 3, block size 10)."""
    cs, cl = [0, 700, 1400], [700, 700, 600]
    wl = custom_workload(seed=41, ctx_len=2000, n_q_heads=6, n_kv_heads=2, block_size=10,
                         anchor=[2000, 350, 1500, 0], ctx_begin=[0, 0, 200, 0], chunk_start=cs,
                         chunk_len=cl, backward=True)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    shape.scale = 0.3
    chunks = bsx.Chunks(cs, cl)
    log("backward, scale 0.3")
    o_part, lse_part = run_fwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"],
                               dev["v_self"], dev["anchor"], dev["ctx_begin"], chunks)
    o, lse = run_merge(o_part, lse_part)
    grads = run_bwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"], o, lse,
                    dev["d_o"], dev["anchor"], dev["ctx_begin"], chunks)
    torch.cuda.synchronize()
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 10, np.asarray(cs), np.asarray(cl),
                                  np.zeros(len(cs), np.int64), 1, scale=0.3)
    nq, hq = wl.q.shape[0], 6
    mo, ml = oracle.lse_merge(ro.reshape(2, nq * hq, -1), rl.reshape(2, nq * hq))
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 10, np.asarray(cs), np.asarray(cl), wl.d_o,
                                  mo.reshape(nq, hq, -1), ml.reshape(nq, hq), scale=0.3)
    for name, got, ref in zip(["dq", "dk", "dv", "dk_self", "dv_self"], grads, r):
        _check(name, got.cpu().numpy(), ref)
