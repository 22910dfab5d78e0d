"""Workload generator checks (CPU only): shapes against the pages' target-model table,
determinism, and the packing rules of the training workload."""
import json
import os

import numpy as np

from workloads import get_config, make_workload
from workloads.gen import round_to_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_head_shapes_match_target_model_table():
    with open(os.path.join(GOLDEN, "target_model_shapes.json")) as f:
        rows = json.load(f)["rows"]
    a3b, b27 = rows
    for i in (1, 3):
        c = get_config(i)
        assert (c.n_q_heads, c.n_kv_heads, c.head_dim) == \
            (a3b["n_q_heads"], a3b["n_kv_heads"], a3b["head_dim"])
    for i in (2, 4):
        c = get_config(i)
        assert (c.n_q_heads, c.n_kv_heads, c.head_dim) == \
            (b27["n_q_heads"], b27["n_kv_heads"], b27["head_dim"])


def test_generation_is_deterministic_and_in_range():
    for cfg in (get_config(n) for n in ("tiny_f32", "a3b_s16k", "b27_s64k")):
        a = make_workload(cfg)
        b = make_workload(cfg)
        np.testing.assert_array_equal(a.anchor, b.anchor)
        np.testing.assert_array_equal(a.q, b.q)
        assert len(np.unique(a.anchor)) == cfg.n_anchors
        assert a.anchor.min() >= cfg.anchor_lo and a.anchor.max() < cfg.anchor_hi
        assert np.all(np.diff(a.anchor) > 0)
        assert a.q.shape == (cfg.n_anchors * cfg.block_size, cfg.n_q_heads, cfg.head_dim)


def test_bf16_rounding_is_exact_and_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.0000001, 65504.0], np.float32)
    r = round_to_bf16(x)
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    assert r[0] == 1.0
    assert r[1] == 1.0            # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0)
    assert r[2] == 1.0078125      # 1 + 1.5 * 2^-8 rounds up
    wl = make_workload(get_config(1))
    assert np.all((wl.q.view(np.uint32) & 0xFFFF) == 0)


def test_training_workload_packing():
    cfg = get_config(4)
    wl = make_workload(cfg)
    assert len(wl.sample_len) == cfg.n_samples
    assert sum(wl.sample_len) <= cfg.ctx_len
    assert all(cfg.len_lo <= n <= cfg.len_hi for n in wl.sample_len)
    n_anchor = sum(n // cfg.anchor_every for n in wl.sample_len)
    assert wl.n_blocks == n_anchor
    for s0, n in zip(wl.sample_start, wl.sample_len):
        sel = wl.ctx_begin == s0
        assert np.all((wl.anchor[sel] >= s0) & (wl.anchor[sel] < s0 + n))
        assert sel.sum() == n // cfg.anchor_every
    k, v = wl.kv_chunks([3, 1])
    k1, _ = wl.kv_chunks([1])
    np.testing.assert_array_equal(k[cfg.chunk_len:], k1)
