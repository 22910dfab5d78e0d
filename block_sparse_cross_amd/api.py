"""Python binding of libbsx, one function per C ABI entry point.

Torch supplies device memory and the current stream; this module only checks that
tensors match the C ABI's layouts (so no call can address past a buffer) and
marshals pointers.  Every step of the computation runs inside libbsx.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

from ._lib import (BSX_BF16, BSX_F32, BsxChunks, BsxError, BsxShape, check, lib)

_DTYPES = {"f32": (BSX_F32, torch.float32), "bf16": (BSX_BF16, torch.bfloat16)}


@dataclass
class Shape:
    n_blocks: int
    block_size: int
    n_q_heads: int
    n_kv_heads: int
    ctx_len: int
    head_dim: int = 128
    dtype: str = "bf16"
    scale: float = 0.0

    @property
    def n_queries(self) -> int:
        return self.n_blocks * self.block_size

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype][1]

    def c(self) -> BsxShape:
        return BsxShape(self.n_blocks, self.block_size, self.n_q_heads, self.n_kv_heads,
                        self.head_dim, _DTYPES[self.dtype][0], self.ctx_len, self.scale)


class Chunks:
    """Host chunk table: chunk i covers packed positions [start[i], start[i] + len[i]) and
    feeds output slot slot[i] (None: slot i).  The local K/V buffer holds the chunks back
    to back in index order."""

    def __init__(self, start: Sequence[int], length: Sequence[int],
                 slot: Optional[Sequence[int]] = None, n_slots: Optional[int] = None):
        self.start = np.ascontiguousarray(start, dtype=np.int64)
        self.length = np.ascontiguousarray(length, dtype=np.int64)
        if self.start.shape != self.length.shape or self.start.ndim != 1:
            raise ValueError("start and length must be 1-D arrays of equal size")
        self.slot = None if slot is None else np.ascontiguousarray(slot, dtype=np.int32)
        if n_slots is None:
            n_slots = len(self.start) if self.slot is None else \
                (int(self.slot.max()) + 1 if len(self.slot) else 0)
        self.n_slots = int(n_slots)

    @property
    def n_chunks(self) -> int:
        return int(self.start.shape[0])

    @property
    def n_local(self) -> int:
        return int(self.length.sum())

    def c(self) -> BsxChunks:
        i64 = ctypes.POINTER(ctypes.c_int64)
        i32 = ctypes.POINTER(ctypes.c_int32)
        return BsxChunks(self.n_chunks, self.n_slots, self.start.ctypes.data_as(i64),
                         self.length.ctypes.data_as(i64),
                         None if self.slot is None else self.slot.ctypes.data_as(i32))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: Optional[torch.Tensor], name: str, shape, dtype, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is None:
        return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
    if ws.numel() < nbytes or ws.dtype != torch.uint8 or not ws.is_cuda:
        raise ValueError(f"workspace needs {nbytes} bytes of uint8 device memory")
    return ws


def abi_version() -> int:
    return int(lib().bsx_abi_version())


def mask_from_anchors(shape: Shape, anchor_global, sample_start=None):
    """-> (ctx_begin, anchor) int64 host arrays: block b sees [ctx_begin[b], anchor[b])
    (bsx_mask_from_anchors)."""
    a = np.ascontiguousarray(anchor_global, dtype=np.int64)
    if a.shape != (shape.n_blocks,):
        raise ValueError("anchor_global must have n_blocks entries")
    s0 = None
    if sample_start is not None:
        s0 = np.ascontiguousarray(sample_start, dtype=np.int64)
        if s0.shape != (shape.n_blocks,):
            raise ValueError("sample_start must have n_blocks entries")
    begin = np.empty(shape.n_blocks, np.int64)
    anchor = np.empty(shape.n_blocks, np.int64)
    i64 = ctypes.POINTER(ctypes.c_int64)
    sc = shape.c()
    check(lib().bsx_mask_from_anchors(ctypes.byref(sc), a.ctypes.data_as(i64),
                                      None if s0 is None else s0.ctypes.data_as(i64),
                                      begin.ctypes.data_as(i64), anchor.ctypes.data_as(i64)))
    return begin, anchor


def validate_mask(shape: Shape, anchor, ctx_begin) -> None:
    a = np.ascontiguousarray(anchor, dtype=np.int64)
    b = np.ascontiguousarray(ctx_begin, dtype=np.int64)
    if a.shape != (shape.n_blocks,) or b.shape != (shape.n_blocks,):
        raise ValueError("anchor/ctx_begin must have n_blocks entries")
    i64 = ctypes.POINTER(ctypes.c_int64)
    sc = shape.c()
    check(lib().bsx_validate_mask(ctypes.byref(sc), a.ctypes.data_as(i64), b.ctypes.data_as(i64)))


@dataclass
class LptResult:
    bin_of: np.ndarray
    loads: np.ndarray
    makespan: int
    imbalance: float


def lpt(cost, n_bins: int) -> LptResult:
    c = np.ascontiguousarray(cost, dtype=np.int64)
    n = int(c.shape[0])
    bin_of = np.empty(n, np.int32)
    loads = np.empty(max(int(n_bins), 0), np.int64)
    ms = ctypes.c_int64(0)
    imb = ctypes.c_double(0.0)
    check(lib().bsx_lpt(n, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), int(n_bins),
                        bin_of.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                        loads.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(ms),
                        ctypes.byref(imb)))
    return LptResult(bin_of, loads, int(ms.value), float(imb.value))


PLACEMENTS = {"lpt": 0, "contiguous": 1, "zigzag": 2, "round_robin": 3}


def place(mode: str, cost, n_bins: int) -> LptResult:
    """Chunk placement by a named rule (bsx_place): lpt, contiguous, zigzag, round_robin."""
    c = np.ascontiguousarray(cost, dtype=np.int64)
    n = int(c.shape[0])
    bin_of = np.empty(n, np.int32)
    loads = np.empty(max(int(n_bins), 0), np.int64)
    ms = ctypes.c_int64(0)
    imb = ctypes.c_double(0.0)
    check(lib().bsx_place(PLACEMENTS[mode], n, c.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                          int(n_bins), bin_of.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                          loads.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(ms),
                          ctypes.byref(imb)))
    return LptResult(bin_of, loads, int(ms.value), float(imb.value))


def cost_workspace_bytes(n_chunks: int) -> int:
    return int(lib().bsx_cost_workspace(int(n_chunks)))


def cost(shape: Shape, anchor: torch.Tensor, ctx_begin: torch.Tensor, chunks: Chunks,
         with_counts: bool = True, ws: Optional[torch.Tensor] = None, out=None,
         _launch: bool = True):
    """-> (counts [n_blocks, n_chunks] int64 or None, chunk_cost [n_chunks] int64, mask_err int32[1])."""
    dev = anchor.device
    _need(anchor, "anchor", (shape.n_blocks,), torch.int64, dev)
    _need(ctx_begin, "ctx_begin", (shape.n_blocks,), torch.int64, dev)
    nc = chunks.n_chunks
    if out is None:
        counts = torch.empty((shape.n_blocks, nc), dtype=torch.int64, device=dev) \
            if with_counts else None
        chunk_cost = torch.empty(nc, dtype=torch.int64, device=dev)
        mask_err = torch.empty(1, dtype=torch.int32, device=dev)
    else:
        counts, chunk_cost, mask_err = out
        if counts is not None:
            _need(counts, "counts", (shape.n_blocks, nc), torch.int64, dev)
        _need(chunk_cost, "chunk_cost", (nc,), torch.int64, dev)
        _need(mask_err, "mask_err", (1,), torch.int32, dev)
    nbytes = cost_workspace_bytes(nc)
    ws = _workspace(nbytes, dev, ws)
    if not _launch:
        return counts, chunk_cost, mask_err
    sc, cc = shape.c(), chunks.c()
    check(lib().bsx_cost(ctypes.byref(sc), _ptr(anchor), _ptr(ctx_begin), ctypes.byref(cc),
                         _ptr(counts), _ptr(chunk_cost), _ptr(mask_err), _ptr(ws),
                         ws.numel(), _stream(anchor)))
    return counts, chunk_cost, mask_err


def fwd_workspace_bytes(shape: Shape, chunks: Chunks) -> int:
    sc, cc = shape.c(), chunks.c()
    return int(lib().bsx_fwd_workspace(ctypes.byref(sc), ctypes.byref(cc)))


def attn_fwd(shape: Shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks: Chunks,
             o_part=None, lse_part=None, ws: Optional[torch.Tensor] = None,
             _launch: bool = True):
    """-> (o_part [n_out, N_q, H_q, d] f32, lse_part [n_out, N_q, H_q] f32)."""
    dev = q.device
    dt = shape.torch_dtype
    nq, hq, hk, d = shape.n_queries, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    _need(q, "q", (nq, hq, d), dt, dev)
    nl = chunks.n_local
    _need(k, "k", (nl, hk, d), dt, dev)
    _need(v, "v", (nl, hk, d), dt, dev)
    if (k_self is None) != (v_self is None):
        raise ValueError("k_self and v_self must both be given or both be None")
    if k_self is not None:
        _need(k_self, "k_self", (nq, hk, d), dt, dev)
        _need(v_self, "v_self", (nq, hk, d), dt, dev)
    _need(anchor, "anchor", (shape.n_blocks,), torch.int64, dev)
    _need(ctx_begin, "ctx_begin", (shape.n_blocks,), torch.int64, dev)
    n_out = chunks.n_slots + (1 if k_self is not None else 0)
    if o_part is None:
        o_part = torch.empty((n_out, nq, hq, d), dtype=torch.float32, device=dev)
    if lse_part is None:
        lse_part = torch.empty((n_out, nq, hq), dtype=torch.float32, device=dev)
    _need(o_part, "o_part", (n_out, nq, hq, d), torch.float32, dev)
    _need(lse_part, "lse_part", (n_out, nq, hq), torch.float32, dev)
    ws = _workspace(fwd_workspace_bytes(shape, chunks), dev, ws)
    if not _launch:
        return o_part, lse_part
    sc, cc = shape.c(), chunks.c()
    check(lib().bsx_attn_fwd(ctypes.byref(sc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_self),
                             _ptr(v_self), _ptr(anchor), _ptr(ctx_begin), ctypes.byref(cc),
                             _ptr(o_part), _ptr(lse_part), _ptr(ws), ws.numel(), _stream(q)))
    return o_part, lse_part


_OUT_DTYPES = {torch.float32: BSX_F32, torch.bfloat16: BSX_BF16}


def lse_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, o_out=None, lse_out=None,
              out_dtype: torch.dtype = torch.float32, _launch: bool = True):
    """o_parts [P, *rows, d], lse_parts [P, *rows] (f32) -> (o [*rows, d], lse [*rows]).

    The merged O is f32, or bf16 (rounded to nearest even) with ``out_dtype`` or a bf16
    ``o_out``."""
    dev = o_parts.device
    P = int(o_parts.shape[0])
    rows_shape = tuple(lse_parts.shape[1:])
    d = int(o_parts.shape[-1])
    n_rows = int(np.prod(rows_shape)) if rows_shape else 1
    _need(o_parts, "o_parts", (P, *rows_shape, d), torch.float32, dev)
    _need(lse_parts, "lse_parts", (P, *rows_shape), torch.float32, dev)
    if o_out is not None:
        out_dtype = o_out.dtype
    if out_dtype not in _OUT_DTYPES:
        raise ValueError(f"merged O dtype {out_dtype} is not float32 or bfloat16")
    if o_out is None:
        o_out = torch.empty((*rows_shape, d), dtype=out_dtype, device=dev)
    if lse_out is None:
        lse_out = torch.empty(rows_shape, dtype=torch.float32, device=dev)
    _need(o_out, "o_out", (*rows_shape, d), out_dtype, dev)
    _need(lse_out, "lse_out", rows_shape, torch.float32, dev)
    if not _launch:
        return o_out, lse_out
    check(lib().bsx_lse_merge(P, n_rows, d, _ptr(o_parts), _ptr(lse_parts),
                              _OUT_DTYPES[out_dtype], _ptr(o_out), _ptr(lse_out),
                              _stream(o_parts)))
    return o_out, lse_out


def bwd_workspace_bytes(shape: Shape, chunks: Chunks) -> int:
    sc, cc = shape.c(), chunks.c()
    return int(lib().bsx_bwd_workspace(ctypes.byref(sc), ctypes.byref(cc)))


def attn_bwd(shape: Shape, q, k, v, k_self, v_self, o, lse, d_o, anchor, ctx_begin,
             chunks: Chunks, out=None, ws: Optional[torch.Tensor] = None,
             _launch: bool = True):
    """-> (dq, dk, dv, dk_self, dv_self), all f32 (dk_self/dv_self None without self keys)."""
    dev = q.device
    dt = shape.torch_dtype
    nq, hq, hk, d = shape.n_queries, shape.n_q_heads, shape.n_kv_heads, shape.head_dim
    nl = chunks.n_local
    _need(q, "q", (nq, hq, d), dt, dev)
    _need(k, "k", (nl, hk, d), dt, dev)
    _need(v, "v", (nl, hk, d), dt, dev)
    if (k_self is None) != (v_self is None):
        raise ValueError("k_self and v_self must both be given or both be None")
    if k_self is not None:
        _need(k_self, "k_self", (nq, hk, d), dt, dev)
        _need(v_self, "v_self", (nq, hk, d), dt, dev)
    _need(o, "o", (nq, hq, d), torch.float32, dev)
    _need(lse, "lse", (nq, hq), torch.float32, dev)
    _need(d_o, "d_o", (nq, hq, d), dt, dev)
    _need(anchor, "anchor", (shape.n_blocks,), torch.int64, dev)
    _need(ctx_begin, "ctx_begin", (shape.n_blocks,), torch.int64, dev)
    f32 = torch.float32
    if out is None:
        dq = torch.empty((nq, hq, d), dtype=f32, device=dev)
        dk = torch.empty((nl, hk, d), dtype=f32, device=dev)
        dv = torch.empty((nl, hk, d), dtype=f32, device=dev)
        dks = torch.empty((nq, hk, d), dtype=f32, device=dev) if k_self is not None else None
        dvs = torch.empty((nq, hk, d), dtype=f32, device=dev) if k_self is not None else None
    else:
        dq, dk, dv, dks, dvs = out
    _need(dq, "dq", (nq, hq, d), f32, dev)
    _need(dk, "dk", (nl, hk, d), f32, dev)
    _need(dv, "dv", (nl, hk, d), f32, dev)
    if k_self is not None:
        _need(dks, "dk_self", (nq, hk, d), f32, dev)
        _need(dvs, "dv_self", (nq, hk, d), f32, dev)
    ws = _workspace(bwd_workspace_bytes(shape, chunks), dev, ws)
    if not _launch:
        return dq, dk, dv, dks, dvs
    sc, cc = shape.c(), chunks.c()
    check(lib().bsx_attn_bwd(ctypes.byref(sc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_self),
                             _ptr(v_self), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(anchor),
                             _ptr(ctx_begin), ctypes.byref(cc), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(dks), _ptr(dvs), _ptr(ws), ws.numel(), _stream(q)))
    return dq, dk, dv, dks, dvs


class Prepared:
    """A validated call of one C ABI entry point: argument checks and pointer
    marshalling ran once; each call re-enters the library with the stored arguments
    on the stream that was current when it was prepared (low host overhead for
    calls repeated every step)."""

    def __init__(self, fn, args: list, keep: list, chunk_slot: Optional[int] = None):
        self._fn = fn
        self._args = args
        # every tensor and ctypes struct the stored arguments point into, held for the
        # life of the call (the arguments are raw addresses)
        self._keep = keep
        self._table = None  # the swapped-in chunk table (host arrays + struct), if any
        self._chunk_slot = chunk_slot

    def set_chunks(self, chunks: "Chunks", like: "Chunks") -> None:
        """Swap the chunk table for another with the same slot count and local length
        (a new plan over the same buffers).  The library reads the table during a call
        only, so the previous swapped-in table is released."""
        if self._chunk_slot is None:
            raise ValueError("this call takes no chunk table")
        if chunks.n_slots != like.n_slots or chunks.n_local != like.n_local:
            raise ValueError("new chunk table does not match the prepared buffers")
        cc = chunks.c()
        self._table = (chunks, cc)
        self._args[self._chunk_slot] = ctypes.byref(cc)

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != 0:
            check(st)


def _prepare(fn, args, keep, chunk_slot=None) -> Prepared:
    return Prepared(fn, list(args), keep, chunk_slot)


def prepare_cost(shape: Shape, anchor, ctx_begin, chunks: Chunks, chunk_cost, mask_err,
                 counts=None, ws=None) -> Prepared:
    dev = anchor.device
    if ws is None:
        raise ValueError("a prepared call needs its workspace")
    cost(shape, anchor, ctx_begin, chunks, with_counts=counts is not None, ws=ws,
         out=(counts, chunk_cost, mask_err), _launch=False)
    ws = _workspace(cost_workspace_bytes(chunks.n_chunks), dev, ws)
    sc, cc = shape.c(), chunks.c()
    args = [ctypes.byref(sc), _ptr(anchor), _ptr(ctx_begin), ctypes.byref(cc), _ptr(counts),
            _ptr(chunk_cost), _ptr(mask_err), _ptr(ws), ws.numel(), _stream(anchor)]
    return _prepare(lib().bsx_cost, args, [sc, cc, chunks, anchor, ctx_begin, counts,
                                           chunk_cost, mask_err, ws], chunk_slot=3)


def prepare_attn_fwd(shape: Shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks: Chunks,
                     o_part, lse_part, ws) -> Prepared:
    attn_fwd(shape, q, k, v, k_self, v_self, anchor, ctx_begin, chunks, o_part, lse_part, ws,
             _launch=False)
    if ws is None:
        raise ValueError("a prepared call needs its workspace")
    sc, cc = shape.c(), chunks.c()
    args = [ctypes.byref(sc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_self), _ptr(v_self), _ptr(anchor),
            _ptr(ctx_begin), ctypes.byref(cc), _ptr(o_part), _ptr(lse_part), _ptr(ws), ws.numel(),
            _stream(q)]
    return _prepare(lib().bsx_attn_fwd, args, [sc, cc, chunks, q, k, v, k_self, v_self, anchor,
                                               ctx_begin, o_part, lse_part, ws], chunk_slot=8)


def prepare_lse_merge(o_parts, lse_parts, o_out, lse_out) -> Prepared:
    lse_merge(o_parts, lse_parts, o_out, lse_out, _launch=False)
    P = int(o_parts.shape[0])
    d = int(o_parts.shape[-1])
    n_rows = int(np.prod(lse_parts.shape[1:])) if lse_parts.dim() > 1 else 1
    args = [P, n_rows, d, _ptr(o_parts), _ptr(lse_parts), _OUT_DTYPES[o_out.dtype], _ptr(o_out),
            _ptr(lse_out), _stream(o_parts)]
    return _prepare(lib().bsx_lse_merge, args, [o_parts, lse_parts, o_out, lse_out])


def prepare_attn_bwd(shape: Shape, q, k, v, k_self, v_self, o, lse, d_o, anchor, ctx_begin,
                     chunks: Chunks, out, ws) -> Prepared:
    attn_bwd(shape, q, k, v, k_self, v_self, o, lse, d_o, anchor, ctx_begin, chunks, out, ws,
             _launch=False)
    if ws is None or out is None:
        raise ValueError("a prepared call needs its outputs and workspace")
    dq, dk, dv, dks, dvs = out
    sc, cc = shape.c(), chunks.c()
    args = [ctypes.byref(sc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_self), _ptr(v_self), _ptr(o),
            _ptr(lse), _ptr(d_o), _ptr(anchor), _ptr(ctx_begin), ctypes.byref(cc), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(dks), _ptr(dvs), _ptr(ws), ws.numel(), _stream(q)]
    return _prepare(lib().bsx_attn_bwd, args, [sc, cc, chunks, q, k, v, k_self, v_self, o, lse,
                                               d_o, anchor, ctx_begin, dq, dk, dv, dks, dvs, ws],
                    chunk_slot=11)


__all__ = ["Prepared", "prepare_cost", "prepare_attn_fwd", "prepare_lse_merge",
           "prepare_attn_bwd", "Shape", "Chunks", "BsxError", "abi_version", "mask_from_anchors", "validate_mask", "lpt", "LptResult",
           "cost", "cost_workspace_bytes", "attn_fwd", "fwd_workspace_bytes", "lse_merge",
           "attn_bwd", "bwd_workspace_bytes"]
