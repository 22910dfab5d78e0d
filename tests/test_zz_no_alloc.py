"""bsx_attn_fwd_noalloc, the forward that allocates nothing (its scratch is a file-scope
device array), against bsx_attn_fwd with a caller workspace, through the C ABI.

Each case runs two calls in a row on the same device, the second on a smaller input,
so the second call must not depend on what the first left in the shared scratch.
Launches that bsx_attn_fwd runs unsplit use the same kernels in the same order and must
match bit for bit; a launch it splits (few KV-head/slot pairs) must match within the
bf16 tolerances.  Outputs are NaN before every call.
"""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_cross_amd as bsx
from block_sparse_cross_amd._lib import BSX_E_UNSUPPORTED, check, lib
from parity_helpers import compare_partials, log, nan_tensor, run_fwd, shape_of, upload
from workloads import get_config, make_workload
from workloads.gen import custom_workload


def _noalloc_fwd(shape, q, k, v, ks, vs, anchor, begin, chunks):
    n_out = chunks.n_slots + (1 if ks is not None else 0)
    nq, hq, d = shape.n_queries, shape.n_q_heads, shape.head_dim
    o = nan_tensor((n_out, nq, hq, d), q.device)
    lse = nan_tensor((n_out, nq, hq), q.device)
    sc, cc = shape.c(), chunks.c()
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    check(lib().bsx_attn_fwd_noalloc(ctypes.byref(sc), p(q), p(k), p(v), p(ks), p(vs), p(anchor),
                                     p(begin), ctypes.byref(cc), p(o), p(lse), stream))
    return o, lse


def _case(name):
    if name == "a3b":  # 17 per-chunk slots, 4 KV heads, launch order over 8 XCD lists
        wl = make_workload(get_config("a3b_s16k"))
        return wl, bsx.Chunks(wl.chunk_start, wl.chunk_len), True, False
    if name == "train_lpt":  # 16 LPT bins of 8 chunks + self slot
        wl = make_workload(get_config("train_pack128k"))
        bins = np.arange(wl.n_chunks) % 16
        return wl, bsx.Chunks(wl.chunk_start, wl.chunk_len, bins, 16), True, False
    if name == "uploaded_table":  # 300 chunks: the table goes through the scratch
        cs, cl = list(range(0, 4800, 16)), [16] * 300
        wl = custom_workload(seed=3, ctx_len=4800, n_q_heads=8, n_kv_heads=2, block_size=16,
                             anchor=[30, 4800, 2400, 1111, 4000], ctx_begin=[0] * 5,
                             chunk_start=cs, chunk_len=cl)
        return wl, bsx.Chunks(cs, cl, np.arange(300) % 7, 7), True, False
    if name == "rank_share":  # 1 fused slot, 4 KV heads: bsx_attn_fwd splits long items
        wl = custom_workload(seed=5, ctx_len=65536, n_q_heads=32, n_kv_heads=4, block_size=16,
                             anchor=[0, 10, 20000, 33000, 50000, 65536], ctx_begin=[0] * 6,
                             chunk_start=[16384, 4096, 40960], chunk_len=[8192] * 3)
        return wl, bsx.Chunks(wl.chunk_start, wl.chunk_len, [0, 0, 0], 1), False, True
    if name == "small":  # a small second input
        wl = custom_workload(seed=9, ctx_len=700, n_q_heads=4, n_kv_heads=4, block_size=5,
                             anchor=[3, 100, 650, 699, 700], ctx_begin=[0] * 5,
                             chunk_start=[0, 350], chunk_len=[350, 350])
        return wl, bsx.Chunks([0, 350], [350, 350]), True, False
    raise KeyError(name)


def _compare(name):
    wl, chunks, with_self, split = _case(name)
    k_loc, v_loc = wl.kv_chunks()
    dev = upload(wl, k_loc, v_loc)
    shape = shape_of(wl)
    ks = dev["k_self"] if with_self else None
    vs = dev["v_self"] if with_self else None
    args = (shape, dev["q"], dev["k"], dev["v"], ks, vs, dev["anchor"], dev["ctx_begin"], chunks)
    o1, l1 = _noalloc_fwd(*args)
    o0, l0 = run_fwd(*args)
    torch.cuda.synchronize()
    log(f"no-alloc forward, {name}: {chunks.n_chunks} chunks, {chunks.n_slots} slots")
    if not split:
        assert torch.equal(l0, l1)
        fin = torch.isfinite(l0)
        assert torch.equal(o0[fin], o1[fin])
    a, b = o1.cpu().numpy(), l1.cpu().numpy()
    compare_partials(a, b, o0.cpu().numpy().astype(np.float64), l0.cpu().numpy().astype(np.float64),
                     2e-2, 2e-3, f"no-alloc vs workspace, {name}")


@pytest.mark.gpu
@pytest.mark.parametrize("first", ["a3b", "train_lpt", "uploaded_table", "rank_share"])
def test_noalloc_forward_matches_workspace_forward_twice(first):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _compare(first)
    _compare("small")  # second call, smaller input, same scratch


def test_noalloc_forward_rejects_tables_beyond_its_limit():
    """Checked before anything touches a device: more chunks than the scratch holds."""
    n = 1025
    shape = bsx.Shape(n_blocks=1, block_size=16, n_q_heads=8, n_kv_heads=2, ctx_len=n * 4)
    ch = bsx.Chunks(np.arange(n) * 4, np.full(n, 4))
    sc, cc = shape.c(), ch.c()
    f = ctypes.c_void_p(0x1000)  # never dereferenced: the call fails its argument checks
    st = lib().bsx_attn_fwd_noalloc(ctypes.byref(sc), f, f, f, None, None, f, f,
                                    ctypes.byref(cc), f, f, None)
    assert st == BSX_E_UNSUPPORTED
    assert b"1024" in lib().bsx_last_error()
