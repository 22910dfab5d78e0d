"""Degenerate inputs through the C ABI against the fp64 oracle: no context chunks (the
draft blocks' own keys only), zero-length chunks and slots without chunks, no draft
blocks at all, and a merge of one partial set.  Every output starts as NaN (workspaces
as 0xFF bytes), so a row the library fails to write cannot pass."""
import numpy as np
import pytest
import torch

import block_sparse_cross_amd as bsx
import oracle
from parity_helpers import (compare_partials, log, run_bwd, run_fwd, run_merge, shape_of,
                            tolerances, upload)
from workloads.gen import custom_workload

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 2e-2   # gradients: max abs error <= 2e-2 * max |reference|
GRAD_L2_REL = 1e-2    # and relative L2 error <= 1e-2 (bf16 operands, f32 accumulation)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _check_grad(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    if got.size == 0:
        return
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    log(f"  {name}: max|ref|={scale:.3g} max err={err:.3g}")
    if scale == 0:
        assert err == 0, f"{name}: {err} where the reference is zero"
        return
    l2 = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= GRAD_MAX_REL * scale, f"{name}: max error {err} > {GRAD_MAX_REL} * {scale}"
    assert l2 <= GRAD_L2_REL, f"{name}: relative L2 error {l2} > {GRAD_L2_REL}"


def _merged_reference(wl, k_loc, v_loc, cs, cl, with_self=True):
    """(O, LSE) of every local chunk as one slot plus (optionally) the draft keys, merged."""
    B, hq = wl.cfg.block_size, wl.cfg.n_q_heads
    n = len(cs)
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, B, np.asarray(cs, np.int64),
                                  np.asarray(cl, np.int64), np.zeros(n, np.int64), 1,
                                  with_self=with_self)
    nq = wl.q.shape[0]
    mo, ml = oracle.lse_merge(ro.reshape(ro.shape[0], nq * hq, -1),
                              rl.reshape(rl.shape[0], nq * hq))
    return mo.reshape(nq, hq, -1), ml.reshape(nq, hq)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_self_keys_only(dtype):
    """No context chunk (n_chunks = n_slots = 0): the one output is the self slot, and the
    merge of that single set returns it unchanged up to rounding."""
    wl = custom_workload(seed=31, ctx_len=4096, n_q_heads=8, n_kv_heads=2, dtype=dtype,
                         sigma=1.0 if dtype == "f32" else 0.5, block_size=16,
                         anchor=[0, 100, 4096], ctx_begin=[0, 0, 0], chunk_start=[],
                         chunk_len=[])
    k_loc, v_loc = wl.kv_chunks()
    assert k_loc.shape[0] == 0
    dev = upload(wl, k_loc, v_loc)
    chunks = bsx.Chunks([], [], [], 0)
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"],
                     dev["anchor"], dev["ctx_begin"], chunks)
    assert tuple(o.shape)[0] == 1
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, np.zeros(0, np.int64), np.zeros(0, np.int64),
                                  np.zeros(0, np.int64), 0)
    tol_o, tol_l = tolerances(dtype)
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "self partial")
    mo, ml = run_merge(o, lse)
    compare_partials(mo.cpu().numpy(), ml.cpu().numpy(), ro[0], rl[0], tol_o, tol_l, "merged")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_zero_length_chunks_and_empty_slots(dtype):
    """Slot 1 has no chunk, slot 2 only a zero-length one: both must come out empty
    (LSE = -inf on every row); slots 0 and 3 against the oracle."""
    cs, cl = [0, 1000, 1000, 2000, 3000], [1000, 0, 1000, 500, 0]
    slot_of, n_slots = [0, 2, 0, 3, 3], 4
    wl = custom_workload(seed=32, ctx_len=3000, n_q_heads=8, n_kv_heads=2, dtype=dtype,
                         sigma=1.0 if dtype == "f32" else 0.5, block_size=16,
                         anchor=[10, 999, 1500, 2600, 3000], ctx_begin=[0] * 5,
                         chunk_start=cs, chunk_len=cl)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"],
                     dev["anchor"], dev["ctx_begin"], bsx.Chunks(cs, cl, slot_of, n_slots))
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, np.asarray(cs), np.asarray(cl),
                                  np.asarray(slot_of), n_slots)
    assert np.isneginf(rl[1]).all() and np.isneginf(rl[2]).all()
    tol_o, tol_l = tolerances(dtype)
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")
    mo, ml = run_merge(o, lse)
    uo, ul = _merged_reference(wl, k_loc, v_loc, cs, cl)
    compare_partials(mo.cpu().numpy(), ml.cpu().numpy(), uo, ul, tol_o, tol_l, "merged")


def test_forward_and_backward_without_blocks():
    """n_blocks = 0: the forward has nothing to write and succeeds; the backward still owns
    the local keys, which no block sees, so dK and dV are exactly zero."""
    cs, cl = [0, 700], [500, 300]
    wl = custom_workload(seed=33, ctx_len=1000, n_q_heads=8, n_kv_heads=2, block_size=16,
                         anchor=[], ctx_begin=[], chunk_start=cs, chunk_len=cl, backward=True)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    chunks = bsx.Chunks(cs, cl)
    o, lse = run_fwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"],
                     dev["anchor"], dev["ctx_begin"], chunks)
    assert tuple(o.shape) == (3, 0, 8, 128) and tuple(lse.shape) == (3, 0, 8)
    empty_o = torch.zeros((0, 8, 128), dtype=torch.float32, device=o.device)
    empty_l = torch.zeros((0, 8), dtype=torch.float32, device=o.device)
    dq, dk, dv, dks, dvs = run_bwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"],
                                   dev["v_self"], empty_o, empty_l, dev["d_o"], dev["anchor"],
                                   dev["ctx_begin"], chunks)
    torch.cuda.synchronize()
    assert dq.numel() == 0 and dks.numel() == 0 and dvs.numel() == 0
    assert tuple(dk.shape) == (800, 2, 128)
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0
    assert not torch.isnan(dk).any() and not torch.isnan(dv).any()


def test_backward_self_keys_only():
    """No context chunk: dQ, dK_self and dV_self come from the draft blocks' own keys, and
    the context gradients are empty tensors."""
    wl = custom_workload(seed=34, ctx_len=2048, n_q_heads=8, n_kv_heads=2, block_size=16,
                         anchor=[0, 512, 2048], ctx_begin=[0, 0, 0], chunk_start=[],
                         chunk_len=[], backward=True)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    chunks = bsx.Chunks([], [], [], 0)
    o_part, lse_part = run_fwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"],
                               dev["v_self"], dev["anchor"], dev["ctx_begin"], chunks)
    o, lse = run_merge(o_part, lse_part)
    dq, dk, dv, dks, dvs = run_bwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"],
                                   dev["v_self"], o, lse, dev["d_o"], dev["anchor"],
                                   dev["ctx_begin"], chunks)
    torch.cuda.synchronize()
    ro, rl = _merged_reference(wl, k_loc, v_loc, [], [])
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 16, np.zeros(0, np.int64),
                                  np.zeros(0, np.int64), wl.d_o, ro, rl)
    for name, got, ref in zip(["dq", "dk", "dv", "dk_self", "dv_self"], [dq, dk, dv, dks, dvs],
                              r):
        _check_grad(name, got.cpu().numpy(), ref)


def test_backward_no_visible_key():
    """No self keys and blocks whose ranges miss every local chunk: every row's LSE is
    -inf, so every gradient is exactly zero (nothing NaN from the empty softmax)."""
    cs, cl = [2000, 2500], [300, 200]
    wl = custom_workload(seed=35, ctx_len=3000, n_q_heads=8, n_kv_heads=2, block_size=16,
                         anchor=[0, 500, 1999], ctx_begin=[0, 0, 0], chunk_start=cs,
                         chunk_len=cl, backward=True)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    chunks = bsx.Chunks(cs, cl, [0, 0], 1)
    o_part, lse_part = run_fwd(shape, dev["q"], dev["k"], dev["v"], None, None, dev["anchor"],
                               dev["ctx_begin"], chunks)
    assert torch.isneginf(lse_part).all()
    o, lse = run_merge(o_part, lse_part)
    assert torch.isneginf(lse).all()
    dq, dk, dv, _, _ = run_bwd(shape, dev["q"], dev["k"], dev["v"], None, None, o, lse,
                               dev["d_o"], dev["anchor"], dev["ctx_begin"], chunks)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(t).any(), f"{name}: NaN"
        assert torch.count_nonzero(t).item() == 0, f"{name}: non-zero"
