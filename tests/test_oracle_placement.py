"""Pins of the oracle's static placements (contiguous, zigzag, round-robin) against closed forms.

Split-KV page, Figures & tables (CP comparison table, load-balancing column) names the
strategies; oracle/placement.py states the reading of each.  On linear costs cost_i = i the
loads have closed forms, and zigzag's pairing of run r with run 2P - 1 - r makes all ranks
equal exactly.
"""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("P,k", [(1, 3), (2, 1), (4, 5), (8, 16), (16, 8), (64, 4)])
def test_zigzag_equalizes_linear_costs(P, k):
    n = 2 * k * P
    cost = list(range(n))
    _, loads, ms, imb = oracle.zigzag(cost, P)
    # run s holds chunks s*k .. s*k+k-1: sum = k*s*k + k(k-1)/2; runs r and 2P-1-r together:
    expect = k * k * (2 * P - 1) + k * (k - 1)
    assert loads == [expect] * P
    assert ms == expect and imb == 0.0


@pytest.mark.parametrize("P,k", [(2, 3), (4, 5), (8, 16), (64, 4)])
def test_contiguous_and_round_robin_linear_closed_forms(P, k):
    n = k * P
    cost = list(range(n))
    total = n * (n - 1) // 2
    b, loads, ms, imb = oracle.contiguous(cost, P)
    assert b == [i // k for i in range(n)]
    assert loads == [k * k * r + k * (k - 1) // 2 for r in range(P)]
    assert ms == loads[-1] and imb == pytest.approx(ms / (total / P) - 1.0, rel=1e-15)
    b, loads, ms, imb = oracle.round_robin(cost, P)
    assert b == [i % P for i in range(n)]
    assert loads == [P * k * (k - 1) // 2 + k * r for r in range(P)]
    assert ms == loads[-1]


@pytest.mark.parametrize("seed", range(6))
def test_placements_are_valid_partitions(seed):
    rng = np.random.default_rng(seed)
    n, P = int(rng.integers(1, 300)), int(rng.integers(1, 70))
    cost = rng.integers(0, 10**9, n).tolist()
    for fn in (oracle.contiguous, oracle.zigzag, oracle.round_robin):
        b, loads, ms, imb = fn(cost, P)
        assert len(b) == n and all(0 <= x < P for x in b)
        assert sum(loads) == sum(cost) and ms == max(loads)
    b, _, _, _ = oracle.contiguous(cost, P)
    assert all(b[i] <= b[i + 1] for i in range(n - 1))  # runs of consecutive chunks
    counts = np.bincount(b, minlength=P)
    assert counts.max() - counts.min() <= 1
    b, _, _, _ = oracle.round_robin(cost, P)
    counts = np.bincount(b, minlength=P)
    assert counts.max() - counts.min() <= 1


def test_placements_degenerate_cases():
    assert oracle.zigzag([5], 1)[1] == [5]
    assert oracle.contiguous([0, 0, 0], 2)[3] == 0.0   # zero total: imbalance 0
    # more ranks than chunks: the extra ranks stay empty
    b, loads, ms, _ = oracle.zigzag([3, 1], 4)
    assert sorted(b) == [0, 3] and ms == 3 and sum(loads) == 4
