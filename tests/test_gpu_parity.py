"""GPU parity: libbsx (through its C ABI) against the fp64 oracle on seeded inputs.

Integers (visible-key counts, chunk costs, LPT plans) must match bit for bit.  Floating
point: max abs error <= 1e-5 on O and LSE for f32 inputs; <= 2e-2 on O and <= 2e-3 on LSE
for bf16 inputs with f32 accumulation, and on O also max|dO| <= 2e-2 max|O| and relative
L2 <= 1e-2 per partial set.  Rows with no visible key must be LSE = -inf on both sides.
Every workload is compared on every row, in the launch configuration the benchmark times
(the oracle of the large ones runs in a pool of worker processes).  Outputs and
workspaces are NaN / 0xFF before every launch, so an unwritten row cannot pass.
"""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_cross_amd as bsx
import oracle
from block_sparse_cross_amd.pipeline import make_plan
import oracle_pool
from parity_helpers import (compare_partials, log, oracle_plan, record, run_fwd, run_merge,
                            shape_of, tolerances, upload)
from workloads import get_config, make_workload
from workloads.gen import custom_workload, draw_merge_sets

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- cost + LPT

@pytest.mark.parametrize("name", ["tiny_f32", "a3b_s16k", "b27_s64k", "rank_p64_s1m", "train_pack128k"])
def test_cost_kernel_bit_exact(name):
    wl = make_workload(get_config(name))
    log(f"cost kernel, workload {wl.cfg.name}: blocks={wl.n_blocks} chunks={wl.n_chunks}")
    shape = shape_of(wl)
    anchor = torch.from_numpy(wl.anchor).cuda()
    begin = torch.from_numpy(wl.ctx_begin).cuda()
    counts, cost, err = bsx.cost(shape, anchor, begin, bsx.Chunks(wl.chunk_start, wl.chunk_len))
    counts2, cost2, _ = bsx.cost(shape, anchor, begin, bsx.Chunks(wl.chunk_start, wl.chunk_len))
    ref_counts, ref_cost = oracle.chunk_costs(wl.anchor, wl.ctx_begin, wl.cfg.block_size,
                                              wl.chunk_start, wl.chunk_len)
    assert np.array_equal(counts.cpu().numpy(), ref_counts)
    assert np.array_equal(cost.cpu().numpy(), ref_cost)
    assert int(err.item()) == 0
    assert torch.equal(counts, counts2) and torch.equal(cost, cost2)


def test_cost_kernel_stress_size_sampled():
    # 65536 blocks x 4096 chunks of 1024 keys (2 GiB of counts): sampled rows against the
    # oracle; every row and the chunk costs against properties that hold at any size
    nb, nc, L = 65536, 4096, 1024
    S = nc * L
    rng = np.random.default_rng(23)
    anchor = rng.integers(0, S + 1, size=nb)
    begin = np.minimum(anchor, rng.integers(0, S + 1, size=nb))
    log(f"cost kernel, {nb} blocks x {nc} chunks")
    shape = bsx.Shape(n_blocks=nb, block_size=16, n_q_heads=32, n_kv_heads=4, ctx_len=S)
    starts, lens = np.arange(nc) * L, np.full(nc, L)
    counts, cost, err = bsx.cost(shape, torch.from_numpy(anchor).cuda(),
                                 torch.from_numpy(begin).cuda(), bsx.Chunks(starts, lens))
    assert int(err.item()) == 0
    sel = np.sort(rng.choice(nb, 8, replace=False))
    ref, _ = oracle.chunk_costs(anchor[sel], begin[sel], 16, starts, lens)
    assert np.array_equal(counts[torch.from_numpy(sel).cuda()].cpu().numpy(), ref)
    # each block's row sums to B times its visible length; chunk costs are column sums
    assert torch.equal(counts.sum(1).cpu(), torch.from_numpy(16 * (anchor - begin)))
    assert torch.equal(counts.sum(0), cost)


def test_cost_kernel_block_groups_full_parity_and_flag():
    # 600 blocks: three groups of 256 blocks, ragged chunks; every count against the
    # oracle, then a bad range in the last group must still raise the flag
    rng = np.random.default_rng(29)
    S, nb = 9000, 600
    cuts = np.sort(rng.integers(0, S + 1, size=70))
    bounds = np.concatenate([[0], cuts, [S]])
    starts, lens = bounds[:-1], np.diff(bounds)
    hi = rng.integers(0, S + 1, size=nb)
    lo = np.minimum(hi, rng.integers(0, S + 1, size=nb))
    log(f"cost kernel, {nb} blocks in groups, {len(starts)} ragged chunks")
    shape = bsx.Shape(n_blocks=nb, block_size=5, n_q_heads=4, n_kv_heads=2, ctx_len=S)
    counts, cost, err = bsx.cost(shape, torch.from_numpy(hi).cuda(), torch.from_numpy(lo).cuda(),
                                 bsx.Chunks(starts, lens))
    rc, rcost = oracle.chunk_costs(hi, lo, 5, starts, lens)
    assert np.array_equal(counts.cpu().numpy(), rc) and np.array_equal(cost.cpu().numpy(), rcost)
    assert int(err.item()) == 0
    bad_hi = hi.copy()
    bad_hi[590] = S + 1
    _, _, err = bsx.cost(shape, torch.from_numpy(bad_hi).cuda(), torch.from_numpy(lo).cuda(),
                         bsx.Chunks(starts, lens))
    assert int(err.item()) == 1


def test_cost_kernel_ragged_chunks_and_bad_mask():
    rng = np.random.default_rng(17)
    S = 5000
    cuts = np.sort(rng.integers(0, S + 1, size=37))
    bounds = np.concatenate([[0], cuts, [S]])
    starts, lens = bounds[:-1], np.diff(bounds)
    hi = rng.integers(0, S + 1, size=300)
    lo = np.minimum(hi, rng.integers(0, S + 1, size=300))
    shape = bsx.Shape(n_blocks=300, block_size=7, n_q_heads=4, n_kv_heads=2, ctx_len=S)
    counts, cost, err = bsx.cost(shape, torch.from_numpy(hi).cuda(), torch.from_numpy(lo).cuda(),
                                 bsx.Chunks(starts, lens))
    rc, rcost = oracle.chunk_costs(hi, lo, 7, starts, lens)
    assert np.array_equal(counts.cpu().numpy(), rc) and np.array_equal(cost.cpu().numpy(), rcost)
    assert int(err.item()) == 0
    bad_hi = hi.copy()
    bad_hi[5] = S + 3
    _, _, err = bsx.cost(shape, torch.from_numpy(bad_hi).cuda(), torch.from_numpy(lo).cuda(),
                         bsx.Chunks(starts, lens))
    assert int(err.item()) == 1
    bad_lo = lo.copy()
    bad_lo[7] = hi[7] + 1
    _, _, err = bsx.cost(shape, torch.from_numpy(hi).cuda(), torch.from_numpy(bad_lo).cuda(),
                         bsx.Chunks(starts, lens))
    assert int(err.item()) == 1


@pytest.mark.parametrize("name", ["b27_s64k", "rank_p64_s1m", "train_pack128k"])
def test_plan_matches_oracle(name):
    wl = make_workload(get_config(name))
    c = wl.cfg
    ref = oracle_plan(wl)
    plan = make_plan(shape_of(wl), wl.chunk_start, wl.chunk_len, c.slot_mode, c.n_bins,
                     torch.from_numpy(wl.anchor).cuda(), torch.from_numpy(wl.ctx_begin).cuda())
    assert np.array_equal(plan.chunk_cost, ref["cost"])
    assert np.array_equal(plan.bin_of, ref["bin_of"])
    assert plan.makespan == ref["makespan"]
    assert plan.imbalance == pytest.approx(ref["imbalance"], abs=1e-15)
    assert np.array_equal(plan.local_chunks, ref["local"])
    log(f"  {c.name}: LPT imbalance {plan.imbalance * 100:.3f}% over {c.n_bins} bins")


# ----------------------------------------------------------------------------- forward

def _run_forward(wl, plan_ref):
    k_loc, v_loc = wl.kv_chunks(plan_ref["local"])
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    starts = wl.chunk_start[plan_ref["local"]]
    lens = wl.chunk_len[plan_ref["local"]]
    chunks = bsx.Chunks(starts, lens, plan_ref["slot_of"], plan_ref["n_slots"])
    with_self = wl.cfg.self_slot
    o, lse = run_fwd(shape, dev["q"], dev["k"], dev["v"],
                     dev["k_self"] if with_self else None,
                     dev["v_self"] if with_self else None,
                     dev["anchor"], dev["ctx_begin"], chunks)
    return dev, k_loc, v_loc, starts, lens, o, lse


def _oracle_partials(wl, k_loc, v_loc, starts, lens, slot_of, n_slots, with_self):
    return oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                wl.ctx_begin, wl.cfg.block_size, starts, lens, slot_of,
                                n_slots, with_self=with_self)


def test_forward_f32_tiny_full():
    wl = make_workload(get_config("tiny_f32"))
    log(f"forward f32, {wl.cfg.name}")
    ref = oracle_plan(wl)
    dev, k_loc, v_loc, starts, lens, o, lse = _run_forward(wl, ref)
    ro, rl = _oracle_partials(wl, k_loc, v_loc, starts, lens, ref["slot_of"], ref["n_slots"], True)
    tol_o, tol_l = tolerances("f32")
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")
    mo, ml = run_merge(o, lse)
    uo, ul = oracle.attention(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor, wl.ctx_begin,
                              wl.cfg.block_size)
    compare_partials(mo.cpu().numpy(), ml.cpu().numpy(), uo, ul, tol_o, tol_l, "merged")


def test_forward_bf16_a3b_full():
    wl = make_workload(get_config("a3b_s16k"))
    log(f"forward bf16, {wl.cfg.name} (all rows)")
    ref = oracle_plan(wl)
    dev, k_loc, v_loc, starts, lens, o, lse = _run_forward(wl, ref)
    o2, lse2 = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"],
                       dev["v_self"], dev["anchor"], dev["ctx_begin"],
                       bsx.Chunks(starts, lens, ref["slot_of"], ref["n_slots"]))
    assert torch.equal(lse, lse2)  # deterministic: no atomics, fixed order
    ro, rl = _oracle_partials(wl, k_loc, v_loc, starts, lens, ref["slot_of"], ref["n_slots"], True)
    tol_o, tol_l = tolerances("bf16")
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")
    mo, ml = run_merge(o, lse)
    uo, ul = oracle.attention(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor, wl.ctx_begin,
                              wl.cfg.block_size)
    compare_partials(mo.cpu().numpy(), ml.cpu().numpy(), uo, ul, tol_o, tol_l, "merged")


@pytest.mark.parametrize("name", ["b27_s64k", "rank_p64_s1m", "train_pack128k"])
def test_forward_bf16_full_size_all_rows(name):
    wl = make_workload(get_config(name))
    c = wl.cfg
    log(f"forward bf16, {c.name} (all rows)")
    ref = oracle_plan(wl)
    dev, k_loc, v_loc, starts, lens, o, lse = _run_forward(wl, ref)
    o_np, lse_np = o.cpu().numpy(), lse.cpu().numpy()
    mo, ml = run_merge(o, lse)
    mo_np, ml_np = mo.cpu().numpy(), ml.cpu().numpy()
    del dev, o, lse, mo, ml
    ro, rl = oracle_pool.slot_partials_all(name, wl.n_blocks, wl.n_queries, c.n_q_heads,
                                           c.head_dim, ref["local"], ref["slot_of"],
                                           ref["n_slots"], c.self_slot)
    tol_o, tol_l = tolerances("bf16")
    compare_partials(o_np, lse_np, ro, rl, tol_o, tol_l, f"{name} partials")
    if c.slot_mode == "rank":
        # one partial: the merge must return it (rows without a visible key stay -inf)
        n = wl.n_queries * c.n_q_heads
        uo, ul = oracle.lse_merge(ro.reshape(1, n, -1), rl.reshape(1, n))
        uo, ul = uo.reshape(ro.shape[1:]), ul.reshape(rl.shape[1:])
    else:
        uo, ul = oracle_pool.merged_all(name, wl.n_blocks, wl.n_queries, c.n_q_heads,
                                        c.head_dim)
    compare_partials(mo_np, ml_np, uo, ul, tol_o, tol_l, f"{name} merged")


def test_forward_launch_order_full():
    """Slots of several chunks (more than 32 key tiles each) take the launch-order pass:
    8 KV heads, 5 slots of 8 chunks, 13 row tiles, items from empty to full; compared in
    full, so an item dropped or run twice by the reordering shows up."""
    S, n_chunks, n_slots = 20480, 40, 5
    rng = np.random.default_rng(21)
    n_blocks = 26
    anchor = rng.integers(0, S + 1, n_blocks)
    anchor[:3] = [0, S, 65]
    begin = np.minimum(rng.integers(0, S // 2, n_blocks), anchor)
    starts = list(range(0, S, S // n_chunks))
    lens = [S // n_chunks] * n_chunks
    wl = custom_workload(seed=22, ctx_len=S, n_q_heads=32, n_kv_heads=8, block_size=16,
                         anchor=anchor.tolist(), ctx_begin=begin.tolist(), chunk_start=starts,
                         chunk_len=lens)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    slot_of = np.arange(n_chunks) % n_slots
    ch = bsx.Chunks(starts, lens, slot_of.tolist(), n_slots)
    log(f"forward bf16, launch-order case: {n_blocks} blocks, {n_slots} slots of 8 chunks")
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"],
                          dev["v_self"], dev["anchor"], dev["ctx_begin"], ch)
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, np.asarray(starts), np.asarray(lens),
                                  slot_of, n_slots, with_self=True)
    tol_o, tol_l = tolerances("bf16")
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")


def test_forward_context_sweep_point_all_rows():
    """One point of the fixed-query-budget context sweep (512 draft queries over S = 2^18 keys,
    LPT over 16 bins), every row."""
    wl = make_workload(get_config("sweep_s262144"))
    c = wl.cfg
    log(f"forward bf16, {c.name} (all rows)")
    ref = oracle_plan(wl)
    dev, k_loc, v_loc, starts, lens, o, lse = _run_forward(wl, ref)
    ro, rl = oracle_pool.slot_partials_all(c.name, wl.n_blocks, wl.n_queries, c.n_q_heads,
                                           c.head_dim, ref["local"], ref["slot_of"],
                                           ref["n_slots"], True)
    tol_o, tol_l = tolerances("bf16")
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")


@pytest.mark.parametrize("with_self", [False, True])
def test_forward_split_pieces_full(with_self):
    """A launch with fewer (KV head, slot) pairs than XCDs and long items: the launch-order
    pass cuts items of more than P = 16 key tiles into pieces and the piece merge combines
    them.  One slot of four 2048-key chunks (non-contiguous, rank-like), 16 anchors; compared
    in full."""
    S = 16384
    rng = np.random.default_rng(31)
    anchor = np.sort(rng.choice(S, 16, replace=False)).astype(np.int64)
    anchor[0], anchor[-1] = 0, S
    begin = np.zeros(16, np.int64)
    begin[5] = 3000  # one block with a late context start
    starts, lens = [2048, 6144, 10240, 14336], [2048] * 4
    hk = 2 if with_self else 4
    wl = custom_workload(seed=32, ctx_len=S, n_q_heads=32, n_kv_heads=hk, block_size=16,
                         anchor=anchor.tolist(), ctx_begin=begin.tolist(), chunk_start=starts,
                         chunk_len=lens)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    ch = bsx.Chunks(starts, lens, [0, 0, 0, 0], 1)
    log(f"forward bf16, split pieces (self slot: {with_self})")
    ks = dev["k_self"] if with_self else None
    vs = dev["v_self"] if with_self else None
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], ks, vs, dev["anchor"],
                          dev["ctx_begin"], ch)
    o2, lse2 = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], ks, vs, dev["anchor"],
                            dev["ctx_begin"], ch)
    assert torch.equal(lse, lse2)  # the order changes no value
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, np.asarray(starts), np.asarray(lens),
                                  np.zeros(4, np.int64), 1, with_self=with_self)
    tol_o, tol_l = tolerances("bf16")
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")


# ----------------------------------------------------------------------------- edge cases

EDGE_CASES = {
    # name: (ctx_len, H_q, H_kv, B, anchors, begins, chunk starts, chunk lens, slot_of, n_slots)
    "ragged_chunks": (3000, 8, 2, 16, [0, 1, 777, 2999, 3000], None,
                      [0, 1000, 1999, 2000], [1000, 999, 1, 1000], None, None),
    "anchor_zero_and_gqa8": (2048, 32, 4, 16, [0, 0, 64, 2048], None,
                             [0, 1024], [1024, 1024], None, None),
    "mha_block5": (700, 4, 4, 5, [3, 100, 650, 699, 700, 0, 350], None,
                   [0, 350], [350, 350], None, None),
    "gqa2_block8": (900, 8, 4, 8, [899, 450, 10], None, [0, 300, 600], [300, 300, 300],
                    [1, 0, 1], 2),
    "packed_samples": (4096, 16, 2, 16, [100, 1500, 1600, 4000, 2500], [0, 0, 1000, 2400, 2400],
                       list(range(0, 4096, 512)), [512] * 8, [0, 1, 2, 0, 1, 2, 0, 1], 3),
    "one_chunk": (1536, 8, 1, 16, [1536, 700], None, [0], [1536], None, None),
    # draft blocks larger than a row tile or a key tile: 80 queries x G = 4 (320 rows),
    # 256 queries x G = 2 (512 rows), self slots of several key tiles
    "block80_gqa4": (3000, 8, 2, 80, [0, 1500, 3000, 2999], None, [0, 1000, 2000],
                     [1000, 1000, 1000], None, None),
    "block256_gqa2": (2048, 4, 2, 256, [700, 2048, 1], [0, 100, 0], [0, 1024], [1024, 1024],
                      None, None),
    # one slot whose chunks are listed out of position order (each slot's list is walked
    # in position order)
    "unsorted_slot": (3000, 8, 2, 16, [0, 1, 777, 2999, 3000, 1999], None,
                      [2000, 0, 1000, 2500], [500, 1000, 1000, 500], [0, 0, 0, 1], 2),
    # query-head groups that do not divide a 32- or 128-row tile (a block's rows and a
    # query's heads straddle tiles), with odd block sizes
    "gqa3_block7": (1800, 6, 2, 7, [0, 5, 900, 1799, 1800, 333, 1200], None,
                    [0, 600, 1200], [600, 600, 600], [0, 1, 0], 2),
    "gqa5_block3": (1000, 10, 2, 3, [1000, 1, 500, 999, 250, 750, 0, 100, 900], None,
                    [0, 250, 500, 750], [250, 250, 250, 250], None, None),
    "gqa7_block33": (2100, 7, 1, 33, [2100, 64, 1000, 2099], [0, 0, 500, 1000],
                     [0, 1100], [1100, 1000], None, None),
    "gqa6_block20": (1500, 12, 2, 20, [1500, 700, 20, 1499, 300], [0, 0, 0, 700, 0],
                     [0, 500, 1000], [500, 500, 500], [1, 0, 1], 2),
    # 300 chunks in 3 slots: the chunk table (4.8 KB) is uploaded to the workspace
    # instead of riding in the kernel arguments
    "many_chunks_uploaded": (4800, 8, 2, 16, [30, 4800, 2400, 1111, 4000, 16], None,
                             list(range(0, 4800, 16)), [16] * 300,
                             [(7 * i) % 3 for i in range(300)], 3),
    # 2100 chunks of 2 keys in 4 slots: more entries than the launch-order pass and the
    # dQ plan keep in LDS (the table is read from memory)
    "many_tiny_chunks": (4200, 4, 2, 4, [0, 4200, 2100, 1, 3333, 777], None,
                         list(range(0, 4200, 2)), [2] * 2100, [i % 4 for i in range(2100)], 4),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", sorted(EDGE_CASES))
def test_forward_edge_cases(case, dtype):
    S, hq, hk, B, an, be, cs, cl, slot_of, n_slots = EDGE_CASES[case]
    log(f"edge case {case} ({dtype})")
    be = [0] * len(an) if be is None else be
    wl = custom_workload(seed=zlib.crc32(case.encode()) % 1000, ctx_len=S, n_q_heads=hq, n_kv_heads=hk,
                         dtype=dtype, sigma=1.0 if dtype == "f32" else 0.5, block_size=B,
                         anchor=an, ctx_begin=be, chunk_start=cs, chunk_len=cl)
    n = len(cs)
    slot_of = np.arange(n) if slot_of is None else np.asarray(slot_of)
    n_slots = n if n_slots is None else n_slots
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    chunks = bsx.Chunks(cs, cl, slot_of, n_slots)
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"],
                          dev["v_self"], dev["anchor"], dev["ctx_begin"], chunks)
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, B, np.asarray(cs), np.asarray(cl), slot_of, n_slots)
    tol_o, tol_l = tolerances(dtype)
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")
    mo, ml = run_merge(o, lse)
    pos = np.concatenate([np.arange(s, s + c) for s, c in zip(cs, cl)])
    k_glob = np.zeros((S, hk, 128), np.float32)
    v_glob = np.zeros((S, hk, 128), np.float32)
    k_glob[pos], v_glob[pos] = k_loc, v_loc
    uo, ul = oracle.attention(wl.q, k_glob, v_glob, wl.k_self, wl.v_self, wl.anchor,
                              wl.ctx_begin, B)
    compare_partials(mo.cpu().numpy(), ml.cpu().numpy(), uo, ul, tol_o, tol_l, "merged")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_overlapping_chunks(dtype):
    """Chunks that share positions (distinct keys at the same positions) in one slot: the
    slot's list is sorted but not disjoint.  Partials against the oracle's."""
    cs, cl = [700, 0, 1500, 600], [1000, 1000, 300, 100]
    slot_of, n_slots = [0, 0, 0, 1], 2
    wl = custom_workload(seed=21, ctx_len=2048, n_q_heads=8, n_kv_heads=2, dtype=dtype,
                         sigma=1.0 if dtype == "f32" else 0.5, block_size=16,
                         anchor=[900, 2048, 1600, 50, 650], ctx_begin=[0] * 5, chunk_start=cs,
                         chunk_len=cl)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"],
                          dev["v_self"], dev["anchor"], dev["ctx_begin"],
                          bsx.Chunks(cs, cl, slot_of, n_slots))
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, np.asarray(cs), np.asarray(cl),
                                  np.asarray(slot_of), n_slots)
    tol_o, tol_l = tolerances(dtype)
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")


def test_forward_rank_share_without_self_and_empty_rows():
    """A non-contiguous rank chunk list fused into one slot, no self keys; blocks whose range
    misses every local chunk must come out as LSE = -inf."""
    wl = custom_workload(seed=5, ctx_len=8192, n_q_heads=32, n_kv_heads=4, block_size=16,
                         anchor=[0, 10, 1000, 3000, 5000, 8192], ctx_begin=[0] * 6,
                         chunk_start=[4096, 1024, 7168], chunk_len=[1024, 1024, 1024])
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    chunks = bsx.Chunks(wl.chunk_start, wl.chunk_len, [0, 0, 0], 1)
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], None, None, dev["anchor"],
                          dev["ctx_begin"], chunks)
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, wl.chunk_start, wl.chunk_len, [0, 0, 0], 1,
                                  with_self=False)
    assert np.isneginf(rl[0, :32]).all()  # blocks 0, 1 see none of the local chunks
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, 2e-2, 2e-3, "rank partial")


def test_forward_sharp_scores():
    """The a3b shape with Q scaled by 4 (exact in bf16): score spread ~4x, so the online
    softmax rescaling is exercised far from the near-uniform regime.  All rows."""
    wl = make_workload(get_config("a3b_s16k"))
    wl.q = wl.q * 4.0
    c = wl.cfg
    ref = oracle_plan(wl)
    dev, k_loc, v_loc, starts, lens, o, lse = _run_forward(wl, ref)
    ro, rl = oracle_pool.slot_partials_all("a3b_s16k", wl.n_blocks, wl.n_queries, c.n_q_heads,
                                           c.head_dim, ref["local"], ref["slot_of"],
                                           ref["n_slots"], True, q_scale=4.0)
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, 2e-2, 2e-3, "sharp partials")


def test_forward_split_item_beyond_16bit_tile_count():
    """A split launch (one KV head, one slot) whose items see more than 65535 key tiles
    (4.3M local keys): every tile must be covered by the pieces.  Q = 0, so every score is 0
    and each row's partial is the mean of its visible V with LSE = log(n)."""
    n_keys = 4_300_000
    S = n_keys
    anchor = np.array([S, S - 30_000], np.int64)
    begin = np.array([0, 20_000], np.int64)
    B, hq, hk = 16, 8, 1
    shape = bsx.Shape(n_blocks=2, block_size=B, n_q_heads=hq, n_kv_heads=hk, ctx_len=S)
    assert (anchor - begin).min() // 64 > 65535
    rng = np.random.default_rng(41)
    from workloads.gen import round_to_bf16
    v_np = round_to_bf16(rng.standard_normal((n_keys, hk, 128), dtype=np.float32))
    log(f"forward bf16, split items of {(anchor - begin).tolist()} keys, Q = 0")
    q = torch.zeros((2 * B, hq, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((n_keys, hk, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.from_numpy(v_np).to(torch.bfloat16).cuda()
    ch = bsx.Chunks([0], [n_keys], [0], 1)
    o, lse = run_fwd(shape, q, k, v, None, None, torch.from_numpy(anchor).cuda(),
                     torch.from_numpy(begin).cuda(), ch)
    o_np, lse_np = o.cpu().numpy(), lse.cpu().numpy()
    del q, k, v, o, lse
    ro = np.zeros((1, 2 * B, hq, 128))
    rl = np.zeros((1, 2 * B, hq))
    for b in range(2):
        lo, hi = oracle.visible_context(anchor, begin, b)
        # one query row suffices: every row of the block has the same (zero) query
        ob, lb = oracle.partial_attention(np.zeros((1, 128)), np.zeros((hi - lo, 128)),
                                          v_np[lo:hi, 0], 1.0 / np.sqrt(128))
        ro[0, b * B:(b + 1) * B] = ob[0]
        rl[0, b * B:(b + 1) * B] = lb[0]
    compare_partials(o_np, lse_np, ro, rl, 2e-2, 2e-3, "split items")


def test_forward_custom_scale():
    wl = custom_workload(seed=8, ctx_len=1000, n_q_heads=8, n_kv_heads=2, block_size=16,
                         anchor=[500, 1000], ctx_begin=[0, 0], chunk_start=[0, 500],
                         chunk_len=[500, 500])
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    shape.scale = 0.3
    o, lse = run_fwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"],
                          dev["anchor"], dev["ctx_begin"], bsx.Chunks(wl.chunk_start, wl.chunk_len))
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, wl.chunk_start, wl.chunk_len, [0, 1], 2,
                                  scale=0.3)
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, 2e-2, 2e-3, "scale 0.3")


# ----------------------------------------------------------------------------- merge

def test_merge_rank_sets_full_size_all_rows():
    """64 seeded partial sets of [2048, 32, 128] (one rank's view at CP size 64), every row
    (the oracle runs on 8192-row pieces)."""
    cfg = get_config("rank_p64_s1m")
    n_rows = 2048 * 32
    log("merge, 64 seeded sets of [2048, 32, 128], all rows")
    o_sets, l_sets = draw_merge_sets(cfg, cfg.n_merge_sets, n_rows, 128)
    o_t = torch.from_numpy(o_sets).cuda()
    l_t = torch.from_numpy(l_sets).cuda()
    mo, ml = run_merge(o_t, l_t)
    got_o, got_l = mo.cpu().numpy(), ml.cpu().numpy()
    del o_t, l_t, mo, ml
    worst_o = worst_l = 0.0
    for r0 in range(0, n_rows, 8192):
        ro, rl = oracle.lse_merge(o_sets[:, r0:r0 + 8192], l_sets[:, r0:r0 + 8192])
        np.testing.assert_allclose(got_l[r0:r0 + 8192], rl, atol=1e-5, rtol=0)
        np.testing.assert_allclose(got_o[r0:r0 + 8192], ro, atol=1e-5, rtol=0)
        worst_o = max(worst_o, float(np.abs(got_o[r0:r0 + 8192] - ro).max()))
        worst_l = max(worst_l, float(np.abs(got_l[r0:r0 + 8192] - rl).max()))
    log(f"  64-set merge: max|dO|={worst_o:.3g} max|dLSE|={worst_l:.3g}")
    record("64-set merge", n=n_rows, o=worst_o, lse=worst_l)


# (the merge runs 16-row workgroups up to 32768 rows and 32-row ones above; both here)
@pytest.mark.parametrize("P,R", [(17, 512 * 32), (64, 1000), (128, 77), (17, 40000)])
def test_merge_bf16_output(P, R):
    """The bf16 merged output is the f32 merged output rounded to nearest even: bit-exact
    against the library's own f32 result rounded, and within one bf16 ulp (plus the f32
    path's own 1e-5 tolerance, which decides the rounding of values near zero) of the
    oracle's fp64 result rounded."""
    from workloads.gen import round_to_bf16
    rng = np.random.default_rng(P * 7 + R)
    o = rng.standard_normal((P, R, 128)).astype(np.float32)
    lse = (rng.standard_normal((P, R)) * 3).astype(np.float32)
    lse[rng.random((P, R)) < 0.3] = -np.inf
    lse[:, 5] = -np.inf  # a row with no partial at all
    ot, lt = torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda()
    mo16, ml16 = run_merge(ot, lt, out_dtype="bf16")
    mo32, ml32 = run_merge(ot, lt)
    assert mo16.dtype == torch.bfloat16
    assert torch.equal(ml16, ml32)
    got = mo16.float().cpu().numpy()
    assert np.array_equal(got, round_to_bf16(mo32.cpu().numpy()))
    ro, rl = oracle.lse_merge(o, lse)
    want = round_to_bf16(ro.astype(np.float32))
    # one bf16 ulp of the rounded value (2^-7 relative to its binade)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(want), 1e-30))[1] - 8)
    assert np.all(np.abs(got - want) <= ulp + 1e-5)
    assert np.all(got[5] == 0) and np.isneginf(ml16.cpu().numpy()[5])


def test_merge_with_empty_partials():
    rng = np.random.default_rng(4)
    P, R, d = 7, 1000, 128
    o = rng.standard_normal((P, R, d)).astype(np.float32)
    lse = (rng.standard_normal((P, R)) * 5).astype(np.float32)
    drop = rng.random((P, R)) < 0.4
    lse[drop] = -np.inf
    o[drop] = np.nan  # unspecified O of an empty partial must never be read
    lse[:, 10] = -np.inf  # a row with no visible key at all
    mo, ml = run_merge(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda())
    ro, rl = oracle.lse_merge(o, lse)
    got_o, got_l = mo.cpu().numpy(), ml.cpu().numpy()
    assert np.isneginf(got_l[10]) and np.all(got_o[10] == 0)
    np.testing.assert_array_equal(np.isneginf(got_l), np.isneginf(rl))
    fin = np.isfinite(rl)
    np.testing.assert_allclose(got_l[fin], rl[fin], atol=1e-5, rtol=0)
    np.testing.assert_allclose(got_o[fin], ro[fin], atol=1e-5, rtol=0)


@pytest.mark.parametrize("P,R,d", [(1, 5, 128), (3, 130, 64), (13, 77, 4), (2, 64, 512), (300, 40, 128),
                                   (150, 33000, 4)])
def test_merge_shapes(P, R, d):
    rng = np.random.default_rng(P * 1000 + R)
    o = rng.standard_normal((P, R, d)).astype(np.float32)
    lse = rng.standard_normal((P, R)).astype(np.float32)
    mo, ml = run_merge(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda())
    ro, rl = oracle.lse_merge(o, lse)
    np.testing.assert_allclose(ml.cpu().numpy(), rl, atol=1e-5, rtol=0)
    np.testing.assert_allclose(mo.cpu().numpy(), ro, atol=1e-5, rtol=0)
