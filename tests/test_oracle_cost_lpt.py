"""Pins for the cost count and the LPT planner of the oracle (CPU only).

Cost: key-by-key enumeration against the closed form B * |[c0, c1) ∩ [lo, hi)| and the
total-work identity.  LPT (Graham's rule, as the Split-KV page's Abstract uses it): brute-force
optimum on tiny instances with Graham's bound LPT <= (4/3 - 1/(3P)) OPT, Graham's tight
instance, hand-worked placements, and the degenerate cases.
"""
import numpy as np
import pytest

import oracle
from workloads import get_config, make_workload


@pytest.mark.parametrize("seed", range(5))
def test_cost_closed_form(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(50, 400))
    nb = int(rng.integers(1, 9))
    B = int(rng.integers(1, 20))
    hi = rng.integers(0, S + 1, size=nb)
    lo = np.minimum(hi, rng.integers(0, S + 1, size=nb))
    cuts = np.sort(rng.integers(0, S + 1, size=int(rng.integers(0, 10))))
    bounds = np.concatenate([[0], cuts, [S]])
    starts, lens = bounds[:-1], np.diff(bounds)
    # non-contiguous extra chunks: arbitrary ranges, possibly overlapping others
    extra_s = rng.integers(0, S, size=3)
    extra_l = rng.integers(0, 40, size=3)
    starts = np.concatenate([starts, extra_s])
    lens = np.concatenate([lens, extra_l])
    counts, cost = oracle.chunk_costs(hi, lo, B, starts, lens)
    for b in range(nb):
        for c in range(len(starts)):
            c0, c1 = int(starts[c]), int(starts[c] + lens[c])
            assert counts[b, c] == B * max(0, min(int(hi[b]), c1) - max(int(lo[b]), c0))
    assert counts.dtype == np.int64 and cost.dtype == np.int64
    np.testing.assert_array_equal(cost, counts.sum(0))
    # the covering chunks account for all visible pairs
    ncov = len(bounds) - 1
    assert counts[:, :ncov].sum() == B * int((hi - lo).sum())


def test_cost_of_workload_uses_int64():
    wl = make_workload(get_config(3))
    counts, cost = oracle.chunk_costs(wl.anchor, wl.ctx_begin, wl.cfg.block_size,
                                      wl.chunk_start, wl.chunk_len)
    assert cost.sum() == wl.cfg.block_size * int((wl.anchor - wl.ctx_begin).sum())
    # pairs x query heads overflow int32 on this workload
    assert cost.sum() * wl.cfg.n_q_heads > 2**31


def test_lpt_hand_examples():
    # [5,3,3,2,2,1] on 2 bins, longest first, ties to the lower bin:
    # 5->b0 [5,0]; 3->b1 [5,3]; 3->b1 [5,6]; 2->b0 [7,6]; 2->b1 [7,8]; 1->b0 [8,8]
    bin_of, loads, makespan, imb = oracle.lpt([5, 3, 3, 2, 2, 1], 2)
    assert bin_of == [0, 1, 1, 0, 1, 0] and loads == [8, 8] and makespan == 8 and imb == 0.0
    # [1,7,4,4,2] on 3 bins: 7->b0 [7,0,0]; 4(idx2)->b1; 4(idx3)->b2 [7,4,4];
    # 2->b1 (tie with b2, lower index) [7,6,4]; 1->b2 [7,6,5]; mean 6 -> imbalance 1/6
    bin_of, loads, makespan, imb = oracle.lpt([1, 7, 4, 4, 2], 3)
    assert bin_of == [2, 0, 1, 2, 1] and loads == [7, 6, 5] and makespan == 7
    assert abs(imb - 1 / 6) < 1e-12


@pytest.mark.parametrize("P", [2, 3, 4, 5])
def test_lpt_graham_tight_instance(P):
    # Graham (1969): jobs 2P-1, 2P-1, 2P-2, 2P-2, ..., P+1, P+1, P, P, P on P machines:
    # LPT makespan 4P-1, optimum 3P.
    jobs = []
    for t in range(2 * P - 1, P, -1):
        jobs += [t, t]
    jobs += [P, P, P]
    _, loads, makespan, _ = oracle.lpt(jobs, P)
    assert makespan == 4 * P - 1
    assert sum(loads) == sum(jobs)
    if P <= 3:
        assert oracle.lpt_makespan_opt(jobs, P) == 3 * P


@pytest.mark.parametrize("seed", range(40))
def test_lpt_within_graham_bound_of_brute_force_optimum(seed):
    rng = np.random.default_rng(seed)
    P = int(rng.integers(2, 5))
    n = int(rng.integers(1, 9 if P <= 3 else 8))
    cost = rng.integers(0, 12, size=n).tolist()
    if seed % 5 == 0:
        cost = [3] * n  # all ties
    bin_of, loads, makespan, _ = oracle.lpt(cost, P)
    opt = oracle.lpt_makespan_opt(cost, P)
    assert 3 * P * makespan <= (4 * P - 1) * opt
    # bin_of is consistent with loads
    check = [0] * P
    for c, j in zip(cost, bin_of):
        check[j] += c
    assert check == loads


def test_lpt_degenerate_cases():
    # n <= P: one item per bin, longest first into the lowest bins
    bin_of, loads, m, imb = oracle.lpt([5, 9, 1], 4)
    assert bin_of == [1, 0, 2] and loads == [9, 5, 1, 0] and m == 9
    # equal costs: round robin by index
    bin_of, *_ = oracle.lpt([2] * 7, 3)
    assert bin_of == [0, 1, 2, 0, 1, 2, 0]
    # all zero: every placement is a tie, so all go to bin 0; imbalance defined as 0
    bin_of, loads, m, imb = oracle.lpt([0, 0, 0], 2)
    assert bin_of == [0, 0, 0] and m == 0 and imb == 0.0
    # empty
    bin_of, loads, m, imb = oracle.lpt([], 3)
    assert bin_of == [] and loads == [0, 0, 0] and m == 0
