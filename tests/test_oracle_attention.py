"""Pins for the oracle's masked attention (CPU only).

The oracle is checked against things other than itself: a pure-Python brute force that
spells the mask out key by key, PyTorch's fp64 scaled-dot-product attention with an explicit
boolean mask (a library routine), and closed forms of softmax attention.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.mask import dense_mask
from workloads.gen import custom_workload


def _tiny(seed=0, S=24, nb=3, B=4, hq=4, hk=2, d=8, anchors=None, begins=None):
    rng = np.random.default_rng(seed)
    if anchors is None:
        anchors = np.sort(rng.choice(S + 1, size=nb, replace=False))
    if begins is None:
        begins = np.zeros(nb, np.int64)
    nq = nb * B
    q = rng.standard_normal((nq, hq, d))
    kc = rng.standard_normal((S, hk, d))
    vc = rng.standard_normal((S, hk, d))
    ks = rng.standard_normal((nq, hk, d))
    vs = rng.standard_normal((nq, hk, d))
    return q, kc, vc, ks, vs, np.asarray(anchors, np.int64), np.asarray(begins, np.int64), B


def _brute(q, kc, vc, ks, vs, anchor, begin, B, scale):
    """Softmax attention one (query, head) at a time, looping over every key position."""
    nq, hq, d = q.shape
    S, hk = kc.shape[0], kc.shape[1]
    grp = hq // hk
    O = np.zeros((nq, hq, d))
    L = np.zeros((nq, hq))
    for qi in range(nq):
        blk = qi // B
        for h in range(hq):
            g = [t for t in range(hk) if t * grp <= h < (t + 1) * grp][0]
            sc, vals = [], []
            for k in range(S):
                if begin[blk] <= k < anchor[blk]:
                    sc.append(scale * sum(q[qi, h, i] * kc[k, g, i] for i in range(d)))
                    vals.append(vc[k, g])
            for j in range(nq):
                if j // B == blk:
                    sc.append(scale * sum(q[qi, h, i] * ks[j, g, i] for i in range(d)))
                    vals.append(vs[j, g])
            m = max(sc)
            lse = m + math.log(sum(math.exp(s - m) for s in sc))
            o = np.zeros(d)
            for s, v in zip(sc, vals):
                o += math.exp(s - lse) * v
            O[qi, h], L[qi, h] = o, lse
    return O, L


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_matches_key_by_key_brute_force(seed):
    q, kc, vc, ks, vs, an, be, B = _tiny(seed)
    scale = 1 / math.sqrt(q.shape[2])
    o, lse = oracle.attention(q, kc, vc, ks, vs, an, be, B)
    ob, lb = _brute(q, kc, vc, ks, vs, an, be, B, scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def test_attention_packed_samples_brute_force():
    # two samples: [0, 10) and [10, 24); blocks of the second sample start at 10
    q, kc, vc, ks, vs, _, _, B = _tiny(5, nb=4)
    an = np.array([3, 10, 15, 24])
    be = np.array([0, 0, 10, 10])
    scale = 1 / math.sqrt(q.shape[2])
    o, lse = oracle.attention(q, kc, vc, ks, vs, an, be, B)
    ob, lb = _brute(q, kc, vc, ks, vs, an, be, B, scale)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


def test_attention_matches_torch_sdpa_with_dense_mask():
    wl = custom_workload(seed=7, ctx_len=300, n_q_heads=8, n_kv_heads=2, head_dim=32,
                         dtype="f32", sigma=1.0, block_size=16,
                         anchor=[0, 37, 150, 151, 300], ctx_begin=[0, 0, 0, 0, 0],
                         chunk_start=[0], chunk_len=[300])
    kc, vc = wl.kv_chunks()
    o, lse = oracle.attention(wl.q, kc, vc, wl.k_self, wl.v_self, wl.anchor, wl.ctx_begin, 16)
    S, nq = 300, wl.n_queries
    mask = torch.from_numpy(dense_mask(wl.anchor, wl.ctx_begin, 16, S))  # [nq, S + nq]
    grp = 4
    keys = torch.from_numpy(np.concatenate([kc, wl.k_self], 0)).double()  # [S+nq, hk, d]
    vals = torch.from_numpy(np.concatenate([vc, wl.v_self], 0)).double()
    keys = keys.repeat_interleave(grp, dim=1).permute(1, 0, 2)  # [hq, S+nq, d]
    vals = vals.repeat_interleave(grp, dim=1).permute(1, 0, 2)
    qq = torch.from_numpy(wl.q).double().permute(1, 0, 2)  # [hq, nq, d]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, attn_mask=mask)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12)
    sc = (qq @ keys.transpose(1, 2)) / math.sqrt(32)
    sc = sc.masked_fill(~mask, float("-inf"))
    ref_lse = torch.logsumexp(sc, dim=-1).permute(1, 0).numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_partial_closed_forms():
    rng = np.random.default_rng(3)
    d = 16
    q = rng.standard_normal((5, d))
    k = rng.standard_normal((1, d))
    v = rng.standard_normal((1, d))
    o, lse = oracle.partial_attention(q, k, v, 0.25)
    np.testing.assert_allclose(o, np.repeat(v, 5, 0), atol=1e-15)   # one key: O = v
    np.testing.assert_allclose(lse, 0.25 * (q @ k.T)[:, 0], atol=1e-14)  # LSE = its score
    # zero query: uniform weights -> O = mean(V), LSE = ln m
    k = rng.standard_normal((9, d))
    v = rng.standard_normal((9, d))
    o, lse = oracle.partial_attention(np.zeros((2, d)), k, v, 0.3)
    np.testing.assert_allclose(o, np.repeat(v.mean(0, keepdims=True), 2, 0), atol=1e-14)
    np.testing.assert_allclose(lse, [math.log(9)] * 2, atol=1e-14)
    # all keys equal: scores constant c -> O = mean(V), LSE = c + ln m
    k = np.repeat(rng.standard_normal((1, d)), 9, 0)
    o, lse = oracle.partial_attention(q, k, v, 0.5)
    c = 0.5 * (q @ k[0])
    np.testing.assert_allclose(o, np.repeat(v.mean(0, keepdims=True), 5, 0), atol=1e-13)
    np.testing.assert_allclose(lse, c + math.log(9), atol=1e-13)
    # empty key set
    o, lse = oracle.partial_attention(q, np.zeros((0, d)), np.zeros((0, d)), 0.5)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_lse_gradient_is_softmax():
    # d LSE / d s_k = P_k, checked by central differences on the scores
    rng = np.random.default_rng(11)
    d, m = 6, 7
    q = rng.standard_normal((1, d))
    k = rng.standard_normal((m, d))
    v = rng.standard_normal((m, d))
    o, lse = oracle.partial_attention(q, k, v, 1.0)
    p = np.exp((q @ k.T)[0] - lse[0])
    for j in range(m):
        for i in range(d):
            e = np.zeros_like(k)
            e[j, i] = 1e-6
            lp = oracle.partial_attention(q, k + e, v, 1.0)[1][0]
            lm = oracle.partial_attention(q, k - e, v, 1.0)[1][0]
            np.testing.assert_allclose((lp - lm) / 2e-6, p[j] * q[0, i], atol=1e-8)
    np.testing.assert_allclose(o[0], p @ v, atol=1e-14)


def test_no_context_block_sees_only_its_own_keys():
    q, kc, vc, ks, vs, _, _, B = _tiny(9, nb=2)
    an = np.array([0, 5])
    be = np.array([0, 5])  # second block: empty range [5, 5)
    o, lse = oracle.attention(q, kc, vc, ks, vs, an, be, B)
    for b in range(2):
        sl = slice(b * B, (b + 1) * B)
        for h in range(q.shape[1]):
            g = h // 2
            ob, lb = oracle.partial_attention(q[sl, h], ks[sl, g], vs[sl, g], 1 / math.sqrt(8))
            np.testing.assert_allclose(o[sl, h], ob, atol=1e-14)
            np.testing.assert_allclose(lse[sl, h], lb, atol=1e-14)


def test_mask_error():
    assert not oracle.mask_error([5, 10], [0, 3], 10)
    assert oracle.mask_error([5, 11], [0, 3], 10)    # anchor beyond the context
    assert oracle.mask_error([5, 2], [0, 3], 10)     # begin after anchor
    assert oracle.mask_error([5, 4], [-1, 3], 10)    # negative begin
    assert not oracle.mask_error([0, 10], [0, 10], 10)  # empty ranges are valid
