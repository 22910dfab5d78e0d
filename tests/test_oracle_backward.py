"""Pins for the oracle's attention gradients (CPU only).

Central finite differences of L = sum(dO * O) in fp64 against every input; PyTorch fp64
autograd of a masked softmax written with library ops; closed-form sums that hold because
each row's softmax weights sum to one; and the split of the keys between ranks.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads.gen import custom_workload


def _setup(seed, S=14, nb=3, B=2, hq=4, hk=2, d=4, anchors=(0, 6, 14), begins=(0, 0, 3)):
    rng = np.random.default_rng(seed)
    nq = nb * B
    q = rng.standard_normal((nq, hq, d))
    kc = rng.standard_normal((S, hk, d))
    vc = rng.standard_normal((S, hk, d))
    ks = rng.standard_normal((nq, hk, d))
    vs = rng.standard_normal((nq, hk, d))
    do = rng.standard_normal((nq, hq, d))
    return q, kc, vc, ks, vs, np.array(anchors), np.array(begins), B, do


def _loss(q, kc, vc, ks, vs, an, be, B, do):
    o, _ = oracle.attention(q, kc, vc, ks, vs, an, be, B)
    return float((o * do).sum())


def _grads(q, kc, vc, ks, vs, an, be, B, do):
    o, lse = oracle.attention(q, kc, vc, ks, vs, an, be, B)
    S = kc.shape[0]
    return oracle.attention_backward(q, kc, vc, ks, vs, an, be, B, [0], [S], do, o, lse)


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_central_differences(seed):
    args = _setup(seed)
    q, kc, vc, ks, vs, an, be, B, do = args
    grads = _grads(*args)
    h = 1e-6
    for ti, t in enumerate([q, kc, vc, ks, vs]):
        num = np.zeros_like(t)
        for idx in np.ndindex(t.shape):
            old = t[idx]
            t[idx] = old + h
            lp = _loss(q, kc, vc, ks, vs, an, be, B, do)
            t[idx] = old - h
            lm = _loss(q, kc, vc, ks, vs, an, be, B, do)
            t[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[ti], num, atol=2e-8, rtol=1e-6)


def test_backward_matches_torch_autograd():
    wl = custom_workload(seed=3, ctx_len=90, n_q_heads=8, n_kv_heads=2, head_dim=16,
                         dtype="f32", sigma=1.0, block_size=4, anchor=[0, 20, 61, 90],
                         ctx_begin=[0, 0, 30, 30], chunk_start=[0], chunk_len=[90],
                         backward=True)
    kc, vc = wl.kv_chunks()
    B, grp, S, nq = 4, 4, 90, wl.n_queries
    o, lse = oracle.attention(wl.q, kc, vc, wl.k_self, wl.v_self, wl.anchor, wl.ctx_begin, B)
    got = oracle.attention_backward(wl.q, kc, vc, wl.k_self, wl.v_self, wl.anchor,
                                    wl.ctx_begin, B, [0], [S], wl.d_o, o, lse)
    mask = torch.from_numpy(oracle.mask.dense_mask(wl.anchor, wl.ctx_begin, B, S))
    tq = torch.tensor(wl.q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(kc, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(vc, dtype=torch.float64, requires_grad=True)
    tks = torch.tensor(wl.k_self, dtype=torch.float64, requires_grad=True)
    tvs = torch.tensor(wl.v_self, dtype=torch.float64, requires_grad=True)
    keys = torch.cat([tk, tks], 0).repeat_interleave(grp, dim=1).permute(1, 0, 2)
    vals = torch.cat([tv, tvs], 0).repeat_interleave(grp, dim=1).permute(1, 0, 2)
    sc = (tq.permute(1, 0, 2) @ keys.transpose(1, 2)) / math.sqrt(16)
    p = torch.softmax(sc.masked_fill(~mask, float("-inf")), dim=-1)
    out = (p @ vals).permute(1, 0, 2)
    (out * torch.from_numpy(wl.d_o).double()).sum().backward()
    for g, t in zip(got, [tq, tk, tv, tks, tvs]):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12)


def test_gradient_sums():
    q, kc, vc, ks, vs, an, be, B, do = _setup(4, S=30, nb=4, B=3, hq=6, hk=2, d=5,
                                               anchors=(2, 11, 30, 30), begins=(0, 0, 12, 30))
    dq, dk, dv, dks, dvs = _grads(q, kc, vc, ks, vs, an, be, B, do)
    grp = 3
    for g in range(2):
        # sum over all keys of dV equals the sum of the group's upstream gradients
        np.testing.assert_allclose(dv[:, g].sum(0) + dvs[:, g].sum(0),
                                   do[:, g * grp:(g + 1) * grp].sum((0, 1)), atol=1e-12)
        # each row's dS sums to zero, so dK sums to zero
        np.testing.assert_allclose(dk[:, g].sum(0) + dks[:, g].sum(0), 0, atol=1e-12)
    # keys nobody sees get no gradient: positions [11, 12) and none of sample 2 beyond 30
    assert np.all(dk[11] == 0) and np.all(dv[11] == 0)


def test_rank_shares_sum_to_full_gradient():
    rng = np.random.default_rng(6)
    q, kc, vc, ks, vs, an, be, B, do = _setup(6, S=40, nb=3, B=2, anchors=(9, 27, 40),
                                               begins=(0, 0, 0))
    full = _grads(q, kc, vc, ks, vs, an, be, B, do)
    o, lse = oracle.attention(q, kc, vc, ks, vs, an, be, B)
    starts = np.arange(0, 40, 8)
    lens = np.full(5, 8)
    owner = rng.integers(0, 3, size=5)
    dq_sum = np.zeros_like(q)
    for r in range(3):
        mine = np.nonzero(owner == r)[0]
        pos = np.concatenate([np.arange(starts[c], starts[c] + 8) for c in mine]) \
            if len(mine) else np.zeros(0, np.int64)
        dq, dk, dv, dks, dvs = oracle.attention_backward(
            q, kc[pos], vc[pos], ks, vs, an, be, B, starts[mine], lens[mine], do, o, lse,
            with_self=(r == 0))
        dq_sum += dq
        np.testing.assert_allclose(dk, full[1][pos], atol=1e-13)
        np.testing.assert_allclose(dv, full[2][pos], atol=1e-13)
    np.testing.assert_allclose(dq_sum, full[0], atol=1e-12)
