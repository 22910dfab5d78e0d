"""The C ABI without a GPU: the library loads, exports every function include/bsx.h declares,
its host-only entry points match the oracle bit for bit, and device entry points reject bad
arguments before launching anything."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_cross_amd as bsx
import oracle
from block_sparse_cross_amd._lib import (BSX_E_INVALID, BSX_E_UNSUPPORTED, BSX_E_WORKSPACE,
                                         BsxChunks, BsxShape, lib)
from workloads import get_config, make_workload

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "bsx.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bsx_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) >= 12
    L = lib()
    for n in names:
        assert hasattr(L, n), n
    assert L.bsx_abi_version() == 2


def test_status_strings():
    L = lib()
    assert L.bsx_status_string(0) == b"BSX_OK"
    assert L.bsx_status_string(3) == b"BSX_E_WORKSPACE"


@pytest.mark.parametrize("name", ["b27_s64k", "rank_p64_s1m", "train_pack128k"])
def test_lpt_matches_oracle_on_workload_costs(name):
    wl = make_workload(get_config(name))
    _, cost = oracle.chunk_costs(wl.anchor, wl.ctx_begin, wl.cfg.block_size, wl.chunk_start,
                                 wl.chunk_len)
    got = bsx.lpt(cost, wl.cfg.n_bins)
    bin_of, loads, ms, imb = oracle.lpt(cost, wl.cfg.n_bins)
    assert got.bin_of.tolist() == bin_of
    assert got.loads.tolist() == loads
    assert got.makespan == ms
    assert got.imbalance == pytest.approx(imb, abs=1e-15)


@pytest.mark.parametrize("seed", range(30))
def test_lpt_matches_oracle_random(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(0, 300))
    P = int(rng.integers(1, 70))
    cost = rng.integers(0, 50 if seed % 3 else 5, size=n) * int(rng.integers(1, 1 << 30))
    got = bsx.lpt(cost, P)
    bin_of, loads, ms, imb = oracle.lpt(cost, P)
    assert got.bin_of.tolist() == bin_of
    assert got.loads.tolist() == loads and got.makespan == ms
    assert got.imbalance == pytest.approx(imb, abs=1e-12)


def test_lpt_rejects_bad_arguments():
    with pytest.raises(bsx.BsxError):
        bsx.lpt([1, 2], 0)
    with pytest.raises(bsx.BsxError):
        bsx.lpt([1, -1], 2)


def test_validate_mask_matches_oracle():
    shape = bsx.Shape(n_blocks=3, block_size=4, n_q_heads=4, n_kv_heads=2, ctx_len=50)
    cases = [([10, 50, 0], [0, 20, 0]), ([10, 51, 0], [0, 20, 0]), ([10, 5, 0], [0, 20, 0]),
             ([10, 50, 0], [-1, 20, 0])]
    for an, be in cases:
        bad = oracle.mask_error(an, be, 50)
        if bad:
            with pytest.raises(bsx.BsxError) as e:
                bsx.validate_mask(shape, an, be)
            assert e.value.status == BSX_E_INVALID
        else:
            bsx.validate_mask(shape, an, be)


@pytest.mark.parametrize("name", ["tiny_f32", "a3b_s16k", "rank_p64_s1m", "train_pack128k"])
def test_mask_from_anchors_matches_oracle(name):
    """Packed anchors and their samples' starts -> each block's context range, bit for bit
    the oracle's visible_context."""
    wl = make_workload(get_config(name))
    c = wl.cfg
    shape = bsx.Shape(n_blocks=wl.n_blocks, block_size=c.block_size, n_q_heads=c.n_q_heads,
                      n_kv_heads=c.n_kv_heads, ctx_len=c.ctx_len)
    sample_start = wl.ctx_begin if c.packed else None
    begin, anchor = bsx.mask_from_anchors(shape, wl.anchor, sample_start)
    for b in range(wl.n_blocks):
        assert (int(begin[b]), int(anchor[b])) == oracle.visible_context(wl.anchor, wl.ctx_begin, b)
    if c.packed:
        # each block's range starts at its own sample's first position
        starts = np.asarray(wl.sample_start)
        sample_of = np.searchsorted(starts, wl.anchor, side="right") - 1
        assert np.array_equal(begin, starts[sample_of])


def test_mask_from_anchors_rejects_bad_ranges_and_writes_nothing():
    shape = bsx.Shape(n_blocks=3, block_size=4, n_q_heads=4, n_kv_heads=2, ctx_len=100)
    i64 = ctypes.POINTER(ctypes.c_int64)
    for an, st in [([10, 101, 5], [0, 0, 0]), ([10, 50, 5], [0, 60, 0]),
                   ([10, 50, 5], [-1, 0, 0])]:
        assert oracle.mask_error(an, st, 100)
        a = np.asarray(an, np.int64)
        s0 = np.asarray(st, np.int64)
        out_b = np.full(3, -7, np.int64)
        out_a = np.full(3, -7, np.int64)
        sc = shape.c()
        assert lib().bsx_mask_from_anchors(ctypes.byref(sc), a.ctypes.data_as(i64),
                                           s0.ctypes.data_as(i64), out_b.ctypes.data_as(i64),
                                           out_a.ctypes.data_as(i64)) == BSX_E_INVALID
        assert np.all(out_b == -7) and np.all(out_a == -7)
    # without sample starts every range begins at 0
    begin, anchor = bsx.mask_from_anchors(shape, [0, 100, 37])
    assert begin.tolist() == [0, 0, 0] and anchor.tolist() == [0, 100, 37]


def test_prepared_call_keeps_its_buffers_alive():
    """A prepared call's arguments are raw addresses: every buffer they point into must stay
    referenced by the call however many chunk tables are swapped in."""
    import gc
    import weakref

    class Buf:
        pass

    bufs = [Buf() for _ in range(12)]
    refs = [weakref.ref(b) for b in bufs]
    call = bsx.Prepared(lambda *a: 0, [0] * 12, list(bufs), chunk_slot=3)
    del bufs
    like = bsx.Chunks([0, 10], [10, 10], [0, 1], 2)
    for i in range(40):
        call.set_chunks(bsx.Chunks([0, 10], [10, 10], [i % 2, 1 - i % 2], 2), like)
    gc.collect()
    assert all(r() is not None for r in refs)
    call()


def _shape(**kw):
    base = dict(n_blocks=2, block_size=16, n_q_heads=8, n_kv_heads=2, head_dim=128, dtype=1,
                ctx_len=1024, scale=0.0)
    base.update(kw)
    return BsxShape(**base)


def _chunks(start, length, slot=None, n_slots=None):
    c = bsx.Chunks(start, length, slot, n_slots)
    return c, c.c()


def _fwd(shape, chunks_c, ws_bytes=1 << 20):
    # Only called with arguments that fail validation: nothing is launched, so the
    # placeholder pointers are never dereferenced.
    f = ctypes.c_void_p(0x1000)
    return lib().bsx_attn_fwd(ctypes.byref(shape), f, f, f, f, f, f, f, ctypes.byref(chunks_c),
                              f, f, f, ws_bytes, None)


def test_forward_rejects_bad_arguments_without_launching():
    cc_keep, cc = _chunks([0, 512], [512, 512])
    assert _fwd(_shape(head_dim=64), cc) == BSX_E_UNSUPPORTED
    assert _fwd(_shape(n_q_heads=6, n_kv_heads=4), cc) == BSX_E_INVALID
    assert _fwd(_shape(dtype=7), cc) == BSX_E_INVALID
    assert _fwd(_shape(block_size=0), cc) == BSX_E_INVALID
    assert _fwd(_shape(n_blocks=-1), cc) == BSX_E_INVALID
    assert _fwd(_shape(ctx_len=-5), cc) == BSX_E_INVALID
    k2, bad_range = _chunks([0, 600], [512, 512])        # runs past S
    assert _fwd(_shape(), bad_range) == BSX_E_INVALID
    k3, neg = _chunks([0, 512], [512, -1])
    assert _fwd(_shape(), neg) == BSX_E_INVALID
    k4, bad_slot = _chunks([0, 512], [512, 512], slot=[0, 2], n_slots=2)
    assert _fwd(_shape(), bad_slot) == BSX_E_INVALID
    k5, no_slot = _chunks([0, 512], [512, 512], None, n_slots=1)
    assert _fwd(_shape(), no_slot) == BSX_E_INVALID
    # self keys: both or neither
    assert lib().bsx_attn_fwd(ctypes.byref(_shape()), 1, 1, 1, 1, None, 1, 1, ctypes.byref(cc),
                              1, 1, 1, 1 << 20, None) == BSX_E_INVALID
    # workspace too small
    need = lib().bsx_fwd_workspace(ctypes.byref(_shape()), ctypes.byref(cc))
    assert need > 0
    assert _fwd(_shape(), cc, ws_bytes=need - 1) == BSX_E_WORKSPACE
    assert b"workspace" in lib().bsx_last_error()


def test_merge_and_cost_reject_bad_arguments():
    L = lib()
    assert L.bsx_lse_merge(0, 10, 128, 1, 1, 0, 1, 1, None) == BSX_E_INVALID
    assert L.bsx_lse_merge(2, 10, 130, 1, 1, 0, 1, 1, None) == BSX_E_INVALID
    assert L.bsx_lse_merge(2, -1, 128, 1, 1, 0, 1, 1, None) == BSX_E_INVALID
    assert L.bsx_lse_merge(2, 10, 128, None, 1, 0, 1, 1, None) == BSX_E_INVALID
    assert L.bsx_lse_merge(2, 10, 128, 1, 1, 5, 1, 1, None) == BSX_E_INVALID   # out dtype
    # a bf16 merged output is one weight pass: at most 128 partials
    assert L.bsx_lse_merge(129, 10, 128, 1, 1, 1, 1, 1, None) == BSX_E_UNSUPPORTED
    assert b"128" in L.bsx_last_error()
    keep, cc = _chunks([0], [1024])
    sh = _shape()
    assert L.bsx_cost(ctypes.byref(sh), 1, 1, ctypes.byref(cc), 1, 1, None, 1, 1 << 20,
                      None) == BSX_E_INVALID
    assert L.bsx_cost(ctypes.byref(sh), 1, 1, ctypes.byref(cc), 1, 1, 1, 1, 8,
                      None) == BSX_E_WORKSPACE
    keep2, bad = _chunks([1000], [100])
    assert L.bsx_cost(ctypes.byref(sh), 1, 1, ctypes.byref(bad), 1, 1, 1, 1, 1 << 20,
                      None) == BSX_E_INVALID


def test_backward_rejects_f32_and_missing_self_grads():
    L = lib()
    keep, cc = _chunks([0], [1024])
    f = 1
    assert L.bsx_attn_bwd(ctypes.byref(_shape(dtype=0)), f, f, f, f, f, f, f, f, f, f,
                          ctypes.byref(cc), f, f, f, f, f, f, 1 << 20, None) == BSX_E_UNSUPPORTED
    assert L.bsx_attn_bwd(ctypes.byref(_shape()), f, f, f, f, f, f, f, f, f, f,
                          ctypes.byref(cc), f, f, f, None, f, f, 1 << 20, None) == BSX_E_INVALID


def test_python_binding_checks_buffer_shapes_on_cpu_tensors():
    import torch
    shape = bsx.Shape(n_blocks=1, block_size=16, n_q_heads=8, n_kv_heads=2, ctx_len=64)
    ch = bsx.Chunks([0], [64])
    q = torch.zeros((16, 8, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsx.attn_fwd(shape, q, q, q, None, None, None, None, ch)


@pytest.mark.parametrize("mode", ["contiguous", "zigzag", "round_robin", "lpt"])
@pytest.mark.parametrize("seed", range(4))
def test_place_matches_oracle_random(mode, seed):
    rng = np.random.default_rng(100 + seed)
    n, P = int(rng.integers(1, 400)), int(rng.integers(1, 80))
    cost = rng.integers(0, 10**12, n)
    got = bsx.place(mode, cost, P)
    fn = {"contiguous": oracle.contiguous, "zigzag": oracle.zigzag,
          "round_robin": oracle.round_robin, "lpt": oracle.lpt}[mode]
    b, loads, ms, imb = fn(cost.tolist(), P)
    assert got.bin_of.tolist() == list(b)
    assert got.loads.tolist() == list(loads) and got.makespan == ms
    assert got.imbalance == pytest.approx(imb, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("name", ["b27_s64k", "rank_p64_s1m", "train_pack128k"])
def test_place_matches_oracle_on_workload_costs(name):
    wl = make_workload(get_config(name))
    _, cost = oracle.chunk_costs(wl.anchor, wl.ctx_begin, wl.cfg.block_size, wl.chunk_start,
                                 wl.chunk_len)
    for mode, fn in [("contiguous", oracle.contiguous), ("zigzag", oracle.zigzag),
                     ("round_robin", oracle.round_robin)]:
        got = bsx.place(mode, cost, wl.cfg.n_bins)
        b, loads, ms, _ = fn(cost.tolist(), wl.cfg.n_bins)
        assert got.bin_of.tolist() == list(b) and got.makespan == ms


def test_place_rejects_bad_mode_and_arguments():
    L = bsx.load_library()
    assert L.bsx_place(7, 0, None, 1, None, None, None, None) == BSX_E_INVALID
    with pytest.raises(bsx.BsxError):
        bsx.place("zigzag", [1, 2], 0)
    with pytest.raises(bsx.BsxError):
        bsx.place("round_robin", [1, -1], 2)
