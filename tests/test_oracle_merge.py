"""Pins for slot partials and the LSE merge (CPU only).

Exactness (Split-KV page, Abstract): merging the partials of any chunking and any
chunk-to-slot map must give unchunked attention.  Checked in fp64 to 1e-12 for random
boundaries, empty and single-key chunks, one chunk, non-contiguous slot maps and a
split of the chunks between ranks.  The merge's algebra is checked on its own.
"""
import math

import numpy as np
import pytest

import oracle
from workloads.gen import custom_workload


def _random_chunking(rng, S, n_cuts):
    cuts = np.sort(rng.integers(0, S + 1, size=n_cuts))
    bounds = np.concatenate([[0], cuts, [S]])
    return bounds[:-1].astype(np.int64), np.diff(bounds).astype(np.int64)


def _wl(seed, S=200, nb=4, hq=4, hk=2, d=16, B=8):
    rng = np.random.default_rng(seed)
    anchors = np.sort(rng.choice(S + 1, size=nb, replace=False))
    return custom_workload(seed=seed, ctx_len=S, n_q_heads=hq, n_kv_heads=hk, head_dim=d,
                           dtype="f32", sigma=1.0, block_size=B, anchor=anchors,
                           ctx_begin=np.zeros(nb, np.int64), chunk_start=[0], chunk_len=[S])


def _flat(o, lse):
    ns = o.shape[0]
    return o.reshape(ns, -1, o.shape[-1]), lse.reshape(ns, -1)


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_any_chunking_equals_unchunked(seed):
    rng = np.random.default_rng(100 + seed)
    wl = _wl(seed)
    S = wl.cfg.ctx_len
    kc, vc = wl.kv_chunks()
    ref_o, ref_l = oracle.attention(wl.q, kc, vc, wl.k_self, wl.v_self, wl.anchor,
                                    wl.ctx_begin, wl.cfg.block_size)
    starts, lens = _random_chunking(rng, S, int(rng.integers(0, 12)))
    # include empty and single-key chunks explicitly
    starts = np.concatenate([starts, [S // 2, S // 3]])
    lens = np.concatenate([lens, [0, 0]])
    n_slots = int(rng.integers(1, 6))
    slot_of = rng.integers(0, n_slots, size=len(starts))
    # the local buffer is the chunks back to back in index order; here chunks are a
    # permutation of the context, so build it by gathering positions
    perm = rng.permutation(len(starts))
    starts, lens, slot_of = starts[perm], lens[perm], slot_of[perm]
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(starts, lens)]).astype(np.int64)
    k_loc, v_loc = kc[pos], vc[pos]
    o, lse = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, wl.cfg.block_size, starts, lens, slot_of, n_slots)
    mo, ml = oracle.lse_merge(*_flat(o, lse))
    np.testing.assert_allclose(mo, ref_o.reshape(-1, ref_o.shape[-1]), atol=1e-12)
    np.testing.assert_allclose(ml, ref_l.reshape(-1), atol=1e-12)


def test_single_chunk_and_per_key_chunks():
    wl = _wl(42, S=40, nb=3)
    kc, vc = wl.kv_chunks()
    ref_o, ref_l = oracle.attention(wl.q, kc, vc, wl.k_self, wl.v_self, wl.anchor,
                                    wl.ctx_begin, wl.cfg.block_size)
    for starts, lens in [([0], [40]), (list(range(40)), [1] * 40)]:
        slot_of = list(range(len(starts)))
        o, lse = oracle.slot_partials(wl.q, kc, vc, wl.k_self, wl.v_self, wl.anchor,
                                      wl.ctx_begin, wl.cfg.block_size, starts, lens, slot_of,
                                      len(starts))
        mo, ml = oracle.lse_merge(*_flat(o, lse))
        np.testing.assert_allclose(mo, ref_o.reshape(-1, ref_o.shape[-1]), atol=1e-12)
        np.testing.assert_allclose(ml, ref_l.reshape(-1), atol=1e-12)


def test_rank_split_partials_merge_to_unchunked():
    """Chunks split between two ranks; each rank fuses its local chunks into one slot."""
    rng = np.random.default_rng(5)
    wl = _wl(5, S=256, nb=5)
    kc, vc = wl.kv_chunks()
    starts = np.arange(0, 256, 32, dtype=np.int64)
    lens = np.full(8, 32, np.int64)
    owner = rng.integers(0, 2, size=8)
    parts_o, parts_l = [], []
    for r in range(2):
        mine = np.nonzero(owner == r)[0]
        pos = np.concatenate([np.arange(starts[c], starts[c] + lens[c]) for c in mine]) \
            if len(mine) else np.zeros(0, np.int64)
        o, lse = oracle.slot_partials(wl.q, kc[pos], vc[pos], wl.k_self, wl.v_self, wl.anchor,
                                      wl.ctx_begin, wl.cfg.block_size, starts[mine], lens[mine],
                                      np.zeros(len(mine), np.int64), 1, with_self=(r == 0))
        fo, fl = _flat(o, lse)
        parts_o.append(fo)
        parts_l.append(fl)
    mo, ml = oracle.lse_merge(np.concatenate(parts_o), np.concatenate(parts_l))
    ref_o, ref_l = oracle.attention(wl.q, kc, vc, wl.k_self, wl.v_self, wl.anchor,
                                    wl.ctx_begin, wl.cfg.block_size)
    np.testing.assert_allclose(mo, ref_o.reshape(-1, ref_o.shape[-1]), atol=1e-12)
    np.testing.assert_allclose(ml, ref_l.reshape(-1), atol=1e-12)


def test_merge_algebra():
    rng = np.random.default_rng(8)
    P, R, d = 5, 7, 4
    o = rng.standard_normal((P, R, d))
    lse = rng.standard_normal((P, R)) * 3
    mo, ml = oracle.lse_merge(o, lse)
    # identity: an all -inf partial (its O is garbage and must not be read)
    o2 = np.concatenate([o, np.full((1, R, d), np.nan)])
    l2 = np.concatenate([lse, np.full((1, R), -np.inf)])
    mo2, ml2 = oracle.lse_merge(o2, l2)
    np.testing.assert_allclose(mo2, mo, atol=1e-14)
    np.testing.assert_allclose(ml2, ml, atol=1e-14)
    # commutativity
    perm = rng.permutation(P)
    mo3, ml3 = oracle.lse_merge(o[perm], lse[perm])
    np.testing.assert_allclose(mo3, mo, atol=1e-13)
    np.testing.assert_allclose(ml3, ml, atol=1e-13)
    # associativity: merge of (merge of first 2, rest)
    ao, al = oracle.lse_merge(o[:2], lse[:2])
    mo4, ml4 = oracle.lse_merge(np.concatenate([ao[None], o[2:]]),
                                np.concatenate([al[None], lse[2:]]))
    np.testing.assert_allclose(mo4, mo, atol=1e-13)
    np.testing.assert_allclose(ml4, ml, atol=1e-13)
    # two equal partials: O unchanged, LSE + ln 2
    mo5, ml5 = oracle.lse_merge(np.stack([o[0], o[0]]), np.stack([lse[0], lse[0]]))
    np.testing.assert_allclose(mo5, o[0], atol=1e-14)
    np.testing.assert_allclose(ml5, lse[0] + math.log(2), atol=1e-14)
    # closed form for two partials: weights are a sigmoid of the LSE difference
    w = 1 / (1 + np.exp(lse[1] - lse[0]))
    np.testing.assert_allclose(oracle.lse_merge(o[:2], lse[:2])[0],
                               w[:, None] * o[0] + (1 - w[:, None]) * o[1], atol=1e-14)
    np.testing.assert_allclose(oracle.lse_merge(o[:2], lse[:2])[1],
                               np.logaddexp(lse[0], lse[1]), atol=1e-14)
    # all partials empty -> (0, -inf)
    mo6, ml6 = oracle.lse_merge(np.full((3, 2, d), np.nan), np.full((3, 2), -np.inf))
    assert np.all(mo6 == 0) and np.all(np.isneginf(ml6))
