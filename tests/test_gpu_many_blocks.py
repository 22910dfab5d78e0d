"""GPU parity with many draft blocks or items against the fp64 oracle: more blocks than
one window of the dK/dV kernel's block compaction (128), than the row-statistics kernel
stages in LDS per pass (1024) and than the launch-order pass keeps in LDS (1024), so the
paths that walk blocks in several windows or read their ranges from memory run; and more
(row tile, output) items than the launch-order pass sorts, so the forward launches in
its natural order.  Small heads and blocks keep the oracle fast."""
import numpy as np
import pytest
import torch

import block_sparse_cross_amd as bsx
import oracle
from parity_helpers import compare_partials, log, run_bwd, run_fwd, run_merge, shape_of, tolerances, upload
from workloads.gen import custom_workload

pytestmark = pytest.mark.gpu

GRAD_MAX_REL = 2e-2   # gradients: max abs error <= 2e-2 * max |reference|
GRAD_L2_REL = 1e-2    # and relative L2 error <= 1e-2


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _anchors(rng, n_blocks, ctx_len):
    """Anchors over the whole context, a few at 0 and at ctx_len."""
    a = rng.integers(0, ctx_len + 1, size=n_blocks).astype(np.int64)
    a[:3] = [0, ctx_len, ctx_len // 2]
    return a


def _check_grad(name, got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    l2 = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    log(f"  {name}: max|ref|={scale:.3g} max err={err:.3g} rel-L2={l2:.3g}")
    if scale == 0:
        assert err == 0, name
        return
    assert err <= GRAD_MAX_REL * scale, f"{name}: max error {err} > {GRAD_MAX_REL} * {scale}"
    assert l2 <= GRAD_L2_REL, f"{name}: relative L2 error {l2} > {GRAD_L2_REL}"


@pytest.mark.parametrize("n_blocks", [300, 1100])
def test_forward_many_blocks(n_blocks):
    """Forward partials (two slots plus self) and the merge, every row."""
    S = 2048
    rng = np.random.default_rng(n_blocks)
    cs, cl = [0, 512, 1024, 1536], [512, 512, 512, 512]
    wl = custom_workload(seed=50 + n_blocks, ctx_len=S, n_q_heads=2, n_kv_heads=1,
                         block_size=2, anchor=_anchors(rng, n_blocks, S),
                         ctx_begin=[0] * n_blocks, chunk_start=cs, chunk_len=cl)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    slot_of = [0, 1, 0, 1]
    log(f"forward, {n_blocks} blocks")
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"],
                     dev["anchor"], dev["ctx_begin"], bsx.Chunks(cs, cl, slot_of, 2))
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 2, np.asarray(cs), np.asarray(cl),
                                  np.asarray(slot_of), 2)
    tol_o, tol_l = tolerances("bf16")
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")
    mo, ml = run_merge(o, lse)
    uo, ul = oracle.attention(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                              wl.ctx_begin, 2)
    compare_partials(mo.cpu().numpy(), ml.cpu().numpy(), uo, ul, tol_o, tol_l, "merged")


@pytest.mark.parametrize("n_blocks", [300, 1100])
def test_backward_many_blocks(n_blocks):
    """dQ, dK, dV and the draft-key gradients, every element."""
    S = 2048
    rng = np.random.default_rng(1000 + n_blocks)
    cs, cl = [1024, 0], [1024, 1024]  # listed out of position order
    wl = custom_workload(seed=60 + n_blocks, ctx_len=S, n_q_heads=4, n_kv_heads=2,
                         block_size=2, anchor=_anchors(rng, n_blocks, S),
                         ctx_begin=[0] * n_blocks, chunk_start=cs, chunk_len=cl,
                         backward=True)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    chunks = bsx.Chunks(cs, cl)
    log(f"backward, {n_blocks} blocks")
    o_part, lse_part = run_fwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"],
                               dev["v_self"], dev["anchor"], dev["ctx_begin"], chunks)
    o, lse = run_merge(o_part, lse_part)
    grads = run_bwd(shape, dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"], o, lse,
                    dev["d_o"], dev["anchor"], dev["ctx_begin"], chunks)
    torch.cuda.synchronize()
    ro, rl = oracle.slot_partials(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 2, np.asarray(cs), np.asarray(cl),
                                  np.zeros(2, np.int64), 1)
    nq, hq = wl.q.shape[0], 4
    mo, ml = oracle.lse_merge(ro.reshape(2, nq * hq, -1), rl.reshape(2, nq * hq))
    r = oracle.attention_backward(wl.q, k_loc, v_loc, wl.k_self, wl.v_self, wl.anchor,
                                  wl.ctx_begin, 2, np.asarray(cs), np.asarray(cl), wl.d_o,
                                  mo.reshape(nq, hq, -1), ml.reshape(nq, hq))
    for name, got, ref in zip(["dq", "dk", "dv", "dk_self", "dv_self"], grads, r):
        _check_grad(name, got.cpu().numpy(), ref)


def test_forward_more_items_than_the_launch_order_pass_takes():
    """32768 one-key slots and the self slot over one row tile: 32769 (row tile, output)
    items, more than the launch-order pass sorts (32768), so the forward launches in its
    natural order.  Every partial against the oracle's attention over its one key."""
    n_keys = 32768
    anchor, begin = [n_keys, 12345], [0, 10000]
    wl = custom_workload(seed=70, ctx_len=n_keys, n_q_heads=1, n_kv_heads=1, block_size=1,
                         anchor=anchor, ctx_begin=begin, chunk_start=list(range(n_keys)),
                         chunk_len=[1] * n_keys)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    chunks = bsx.Chunks(np.arange(n_keys), np.ones(n_keys, np.int64))
    log("forward, 32769 items")
    o, lse = run_fwd(shape_of(wl), dev["q"], dev["k"], dev["v"], dev["k_self"], dev["v_self"],
                     dev["anchor"], dev["ctx_begin"], chunks)
    scale = oracle.default_scale(128)
    ro = np.full((n_keys + 1, 2, 1, 128), np.nan)
    rl = np.full((n_keys + 1, 2, 1), np.nan)
    for b in range(2):
        q = wl.q[b:b + 1, 0]
        for s in range(n_keys):
            if begin[b] <= s < anchor[b]:
                ob, lb = oracle.partial_attention(q, k_loc[s:s + 1, 0], v_loc[s:s + 1, 0], scale)
                ro[s, b, 0], rl[s, b, 0] = ob[0], lb[0]
            else:
                rl[s, b, 0] = -np.inf
        ob, lb = oracle.partial_attention(q, wl.k_self[b:b + 1, 0], wl.v_self[b:b + 1, 0], scale)
        ro[n_keys, b, 0], rl[n_keys, b, 0] = ob[0], lb[0]
    tol_o, tol_l = tolerances("bf16")
    compare_partials(o.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_o, tol_l, "partials")
