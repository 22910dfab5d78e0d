"""Benchmark of the draft-query block-sparse cross-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole hot path over one batch of synthetic inputs that
are already resident in HBM: the per-chunk cost kernel, the LPT plan (host, after
the one readback of chunk costs) for planned workloads, the forward partials, the
exact LSE merge, and for the training workload the backward pass.  Steps are
pipelined as a training loop runs them: each batch is planned (cost kernel and cost
readback on a second stream, then the host LPT) while the previous batch's attention
runs, so every timed step does one whole plan and one whole attention pass.  The
default workload is the largest one that runs the whole path, forward and backward:
the packed training step (8 samples packed into 131072 keys, the tail past them
padding that no query sees, H_q = 32, H_kv = 8, d = 128, one anchor per 1024 tokens of
a sample with 16 draft queries each, 128 KV chunks of 1024 balanced by LPT over 16
bins, plus the draft blocks' own keys).

Prints one JSON line: useful TFLOP/s (masked-out and padded work excluded) of the
step; a roofline object for the dominant call (the backward on the training step,
else the forward), timed with HIP events on the stream it runs on; forward rooflines
of the step's workload and of the two other large forward workloads; the standalone
64-set merge against HBM bandwidth; and the fp64 oracle timed on host cores on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "useful TFLOP/s of block-sparse cross-attn fwd (+bwd) and % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 matrix-core peak (the f32 path runs f32 MFMA)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="train_pack128k")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle's CPU baseline sample (0 skips it)")
    ap.add_argument("--fwd-reps", type=int, default=50,
                    help="event-timed launches of the forward kernel for the roofline")
    ap.add_argument("--sweep", action="store_true",
                    help="print the fixed-query-budget context sweep (S = 16K .. 1M) and exit")
    ap.add_argument("--cost-stress", action="store_true",
                    help="time the cost kernel at 65536 blocks x 4096 chunks and exit")
    ap.add_argument("--planners", action="store_true",
                    help="print the chunk-placement comparison (imbalance, host us) and exit")
    ap.add_argument("--no-merge-bench", action="store_true",
                    help="skip the standalone 64-set merge measurement")
    ap.add_argument("--no-extra-fwd", action="store_true",
                    help="skip the forward rooflines of the other large workloads")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a reference "
                         "dispatch for scaling HBM byte counters)")
    return ap.parse_args()


def useful_fwd_flops(wl, with_self: bool) -> float:
    c = wl.cfg
    vis = float((wl.anchor - wl.ctx_begin).sum()) * c.block_size
    if with_self:
        vis += wl.n_blocks * c.block_size * c.block_size
    return 4.0 * c.head_dim * c.n_q_heads * vis


def rank_fwd_flops(wl, local_chunks) -> float:
    """Useful flops of one rank's share: visible (query, key) pairs in its local chunks."""
    c = wl.cfg
    tot = 0.0
    for ch in local_chunks:
        c0 = int(wl.chunk_start[ch])
        c1 = c0 + int(wl.chunk_len[ch])
        ov = np.clip(np.minimum(wl.anchor, c1) - np.maximum(wl.ctx_begin, c0), 0, None)
        tot += float(ov.sum()) * c.block_size
    return 4.0 * c.head_dim * c.n_q_heads * tot


class Step:
    """Device-resident inputs, preallocated outputs and workspaces, and one-step runner."""

    def __init__(self, wl, device, device_kv: bool = False):
        import torch

        import block_sparse_cross_amd as bsx
        from block_sparse_cross_amd.pipeline import make_plan

        self.torch, self.bsx, self.make_plan = torch, bsx, make_plan
        self.wl, self.cfg, self.dev = wl, wl.cfg, device
        c = wl.cfg
        self.shape = bsx.Shape(n_blocks=wl.n_blocks, block_size=c.block_size,
                               n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads, ctx_len=c.ctx_len,
                               head_dim=c.head_dim, dtype=c.dtype)
        dt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
        up = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dt).to(device)  # noqa: E731
        self.anchor = torch.from_numpy(wl.anchor).to(device)
        self.begin = torch.from_numpy(wl.ctx_begin).to(device)
        self.all_chunks = bsx.Chunks(wl.chunk_start, wl.chunk_len)
        self.cost_ws = torch.empty(bsx.cost_workspace_bytes(wl.n_chunks), dtype=torch.uint8,
                                   device=device)
        self.cost_out = (None, torch.empty(wl.n_chunks, dtype=torch.int64, device=device),
                         torch.empty(1, dtype=torch.int32, device=device))
        # plan once to learn which chunks are local (deterministic: every step replans the same)
        self.plan0 = make_plan(self.shape, wl.chunk_start, wl.chunk_len, c.slot_mode, c.n_bins,
                               self.anchor, self.begin, self.cost_ws, self.cost_out)
        if device_kv:
            # timing only: context K/V drawn on the device (seeded), not on the host
            n_loc = int(np.sum(wl.chunk_len[self.plan0.local_chunks]))
            g = torch.Generator(device=device)
            g.manual_seed(c.seed)
            kv_shape = (n_loc, c.n_kv_heads, c.head_dim)
            self.k = (torch.randn(kv_shape, generator=g, device=device) * c.sigma).to(dt)
            self.v = (torch.randn(kv_shape, generator=g, device=device) * c.sigma).to(dt)
            self.q = up(wl.q)
        else:
            k, v = wl.kv_chunks(self.plan0.local_chunks)
            self.q, self.k, self.v = up(wl.q), up(k), up(v)
        self.ks = up(wl.k_self) if c.self_slot else None
        self.vs = up(wl.v_self) if c.self_slot else None
        ch = self.plan0.chunks
        n_out = ch.n_slots + (1 if c.self_slot else 0)
        nq = wl.n_queries
        self.o_part = torch.empty((n_out, nq, c.n_q_heads, c.head_dim), dtype=torch.float32,
                                  device=device)
        self.lse_part = torch.empty((n_out, nq, c.n_q_heads), dtype=torch.float32, device=device)
        self.fwd_ws = torch.empty(max(bsx.fwd_workspace_bytes(self.shape, ch), 256),
                                  dtype=torch.uint8, device=device)
        self.o = torch.empty((nq, c.n_q_heads, c.head_dim), dtype=torch.float32, device=device)
        self.lse = torch.empty((nq, c.n_q_heads), dtype=torch.float32, device=device)
        self.backward = c.backward
        if self.backward:
            self.d_o = up(wl.d_o)
            nl = ch.n_local
            f32 = torch.float32
            self.grads = (torch.empty((nq, c.n_q_heads, c.head_dim), dtype=f32, device=device),
                          torch.empty((nl, c.n_kv_heads, c.head_dim), dtype=f32, device=device),
                          torch.empty((nl, c.n_kv_heads, c.head_dim), dtype=f32, device=device),
                          torch.empty((nq, c.n_kv_heads, c.head_dim), dtype=f32, device=device),
                          torch.empty((nq, c.n_kv_heads, c.head_dim), dtype=f32, device=device))
            self.bwd_ws = torch.empty(max(bsx.bwd_workspace_bytes(self.shape, ch), 256),
                                      dtype=torch.uint8, device=device)
        if c.slot_mode == "rank":
            self.fwd_flops = rank_fwd_flops(wl, self.plan0.local_chunks)
        else:
            self.fwd_flops = useful_fwd_flops(wl, c.self_slot)
        self.step_flops = self.fwd_flops * (3.5 if self.backward else 1.0)

    def prepare(self):
        """Validated, marshalled calls for the per-step launches (low host overhead)."""
        bsx, torch = self.bsx, self.torch
        # the planning of a batch (cost kernel, cost readback, host LPT) runs on a side
        # stream so that it overlaps the previous batch's attention on the main stream
        self.side = torch.cuda.Stream(self.dev)
        with torch.cuda.stream(self.side):
            self.cost_call = bsx.prepare_cost(self.shape, self.anchor, self.begin,
                                              self.all_chunks, self.cost_out[1], self.cost_out[2],
                                              ws=self.cost_ws)
        self.cost_host = torch.empty(self.cost_out[1].shape, dtype=torch.int64, pin_memory=True)
        self.err_host = torch.empty(1, dtype=torch.int32, pin_memory=True)
        self.cost_ready = torch.cuda.Event()
        self.pending_err = False
        self.next_chunks = None
        self.fwd_call = bsx.prepare_attn_fwd(self.shape, self.q, self.k, self.v, self.ks, self.vs,
                                             self.anchor, self.begin, self.plan0.chunks,
                                             self.o_part, self.lse_part, self.fwd_ws)
        self.merge_call = bsx.prepare_lse_merge(self.o_part, self.lse_part, self.o, self.lse)
        self.bwd_call = None
        if self.backward:
            self.bwd_call = bsx.prepare_attn_bwd(self.shape, self.q, self.k, self.v, self.ks,
                                                 self.vs, self.o, self.lse, self.d_o, self.anchor,
                                                 self.begin, self.plan0.chunks, self.grads,
                                                 self.bwd_ws)

    def plan(self):
        """Plans one batch: the cost kernel on the side stream, then (planned workloads)
        readback of the chunk costs into pinned memory and the host LPT.  Returns the
        batch's chunk table (None: the table does not depend on the costs)."""
        c, torch = self.cfg, self.torch
        self.cost_call()
        with torch.cuda.stream(self.side):
            if c.slot_mode != "per_chunk":
                self.cost_host.copy_(self.cost_out[1], non_blocking=True)
            self.err_host.copy_(self.cost_out[2], non_blocking=True)
            self.cost_ready.record(self.side)
        if c.slot_mode == "per_chunk":
            # one partial per chunk: the plan does not depend on the costs; the mask
            # flag of this batch is checked when the next batch is planned
            if self.pending_err and int(self.err_host[0]) != 0:
                raise RuntimeError("cost kernel flagged a block range outside the context")
            self.pending_err = True
            return None
        self.cost_ready.synchronize()
        if int(self.err_host[0]) != 0:
            raise RuntimeError("cost kernel flagged a block range outside the context")
        r = self.bsx.lpt(self.cost_host.numpy(), c.n_bins)
        wl = self.wl
        if c.slot_mode == "lpt":
            return self.bsx.Chunks(wl.chunk_start, wl.chunk_len, r.bin_of, c.n_bins)
        rank = int(np.argmax(r.loads))
        mine = np.nonzero(r.bin_of == rank)[0]
        if not np.array_equal(mine, self.plan0.local_chunks):
            raise RuntimeError("plan changed between steps")
        return self.bsx.Chunks(wl.chunk_start[mine], wl.chunk_len[mine],
                               np.zeros(len(mine), np.int32), 1)

    def use(self, chunks):
        if chunks is None:
            return
        self.fwd_call.set_chunks(chunks, self.plan0.chunks)
        if self.bwd_call is not None:
            self.bwd_call.set_chunks(chunks, self.plan0.chunks)

    def forward(self, chunks=None):
        self.fwd_call()

    def merge(self):
        self.merge_call()

    def run(self):
        """One step: the batch's attention (forward, merge, backward) with the plan made
        for it, then the next batch's plan while that work runs on the GPU.  The first
        call plans its own batch first."""
        if self.next_chunks is None:
            self.next_chunks = (self.plan(),)
        self.use(self.next_chunks[0])
        self.fwd_call()
        self.merge_call()
        if self.bwd_call is not None:
            self.bwd_call()
        self.next_chunks = (self.plan(),)


def time_call(step: Step, fn, reps: int):
    """Average duration of one call of ``fn`` (launches on the current stream), from HIP
    events recorded on that stream around ``reps`` back-to-back calls."""
    torch = step.torch
    stream = torch.cuda.current_stream()
    for _ in range(3):
        fn()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps * 1e-3


def time_forward(step: Step, reps: int):
    return time_call(step, step.forward, reps)


FWD_KERNELS = ["fwd_order_kernel", "fwd_bf16_kernel", "fwd_piece_merge_kernel (split launches)"]
BWD_KERNELS = ["bwd_delta_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel", "bwd_dq_reduce_kernel"]


def fwd_roofline(step: Step, reps: int, workload: str) -> dict:
    """The forward call (launch-order pass + attention kernel [+ piece merge]): useful
    forward FLOPs per call over its average duration."""
    s = time_forward(step, reps)
    f32 = step.cfg.dtype == "f32"
    peak = PEAK_F32_TFLOPS if f32 else PEAK_BF16_TFLOPS
    achieved = step.fwd_flops / s / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": None if f32 else recorded_traffic("fwd", workload),
            "kernel": "fwd_f32_kernel" if f32 else "bsx_attn_fwd: " + " + ".join(FWD_KERNELS),
            "launch_us": round(s * 1e6, 2), "flops_per_launch": step.fwd_flops}


def bwd_roofline(step: Step, reps: int, workload: str) -> dict:
    """The backward call (all of its kernels): useful backward FLOPs (2.5x the forward's:
    S recompute, dP, dV, dK, dQ over the visible pairs) over its average duration."""
    s = time_call(step, step.bwd_call, reps)
    flops = 2.5 * step.fwd_flops
    achieved = flops / s / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": recorded_traffic("bwd", workload),
            "kernel": "bsx_attn_bwd: " + " + ".join(BWD_KERNELS),
            "launch_us": round(s * 1e6, 2), "flops_per_launch": flops}


def merge_bench(device, n_sets: int = 64, rows=(2048, 32), head_dim: int = 128, reps: int = 10,
                seed: int = 4):
    """The standalone exact merge of one rank's view at CP size 64: n_sets seeded partial
    (O, LSE) sets (O ~ N(0,1), LSE ~ N(0,1) + 8, drawn on the device), HBM-bound.
    Algorithmic bytes per launch: every partial row and LSE read once, the merged row written."""
    import torch
    import block_sparse_cross_amd as bsx
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    o = torch.randn((n_sets, *rows, head_dim), generator=g, device=device, dtype=torch.float32)
    lse = torch.randn((n_sets, *rows), generator=g, device=device, dtype=torch.float32) + 8.0
    out_o = torch.empty((*rows, head_dim), device=device, dtype=torch.float32)
    out_l = torch.empty(rows, device=device, dtype=torch.float32)
    call = bsx.prepare_lse_merge(o, lse, out_o, out_l)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=device)  # 512 MiB > infinity cache
    call()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * reps)]
    for i in range(reps):
        flush.zero_()  # cold: the partials are not resident in the infinity cache
        ev[2 * i].record()
        call()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    ts = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e-3 for i in range(reps))
    t = ts[len(ts) // 2]
    n_rows = rows[0] * rows[1]
    nbytes = n_sets * n_rows * (head_dim + 1) * 4 + n_rows * (head_dim + 1) * 4
    del o, lse, flush
    return {"kernel": "lse_merge_kernel", "sets": n_sets, "shape": [*rows, head_dim],
            "bound": "hbm", "bytes_per_launch": nbytes, "launch_us": round(t * 1e6, 2),
            "achieved": round(nbytes / t / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)}


def _host_cpus():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(wl, plan0, seconds: float):
    """The fp64 oracle as it stands, on (block, KV head) pairs taken in a fixed seeded order
    until the time budget is spent: forward partials of every slot and their merge, and for
    training workloads the backward of the same rows (from the oracle's own unchunked
    forward).  Useful TFLOP/s of that sample (the step's flop count restricted to it)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    c = wl.cfg
    k, v = wl.kv_chunks(plan0.local_chunks)
    ch = plan0.chunks
    slot_of = np.arange(ch.n_chunks) if ch.slot is None else ch.slot
    rng = np.random.default_rng(0)
    pairs = [(b, g) for b in range(wl.n_blocks) for g in range(c.n_kv_heads)]
    order = rng.permutation(len(pairs))
    grp = c.group
    B = c.block_size
    done_flops, n_done = 0.0, 0
    t0 = time.perf_counter()
    for idx in order:
        b, g = pairs[idx]
        o, lse = oracle.slot_partials(wl.q, k, v, wl.k_self, wl.v_self, wl.anchor, wl.ctx_begin,
                                      B, ch.start, ch.length, slot_of, ch.n_slots,
                                      with_self=c.self_slot, blocks=[b], groups=[g])
        sl = (slice(None), slice(b * B, (b + 1) * B), slice(g * grp, (g + 1) * grp))
        oracle.lse_merge(o[sl].reshape(o.shape[0], -1, o.shape[-1]),
                         lse[sl].reshape(lse.shape[0], -1))
        vis = 0
        for s0, n in zip(ch.start, ch.length):
            vis += max(0, min(int(wl.anchor[b]), s0 + n) - max(int(wl.ctx_begin[b]), s0))
        if c.self_slot:
            vis += B
        flops = 4.0 * c.head_dim * grp * B * vis
        if c.backward:
            # the block's rows only: the oracle over a one-block view of the inputs
            one = slice(b * B, (b + 1) * B)
            ub, ul = oracle.attention(wl.q[one], k, v, wl.k_self[one], wl.v_self[one],
                                      wl.anchor[b:b + 1], wl.ctx_begin[b:b + 1], B, groups=[g])
            oracle.attention_backward(wl.q[one], k, v, wl.k_self[one], wl.v_self[one],
                                      wl.anchor[b:b + 1], wl.ctx_begin[b:b + 1], B, ch.start,
                                      ch.length, wl.d_o[one], np.nan_to_num(ub),
                                      np.nan_to_num(ul, nan=0.0), groups=[g])
            flops *= 3.5
        done_flops += flops
        n_done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    what = "forward partials of all %d slots + merge%s" % (
        ch.n_slots + int(c.self_slot), " + backward (dQ, dK, dV)" if c.backward else "")
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s",
            "cores": int(min(blas_threads, _host_cpus())), "host_cpus": _host_cpus(),
            "kind": "oracle",
            "sample": f"fp64 oracle {what} for {n_done} of {len(pairs)} (block, KV head) pairs "
                      f"of the same workload, {dt:.1f} s; cores = the BLAS threads it ran on"}


# Sources of each call's kernels; a recorded HBM traffic figure is valid only while they
# are unchanged (of the shared internal header, only the declarations the kernels read).
CALL_SOURCES = {
    "fwd": ["block_sparse_cross_amd/csrc/fwd_bf16.hip", "block_sparse_cross_amd/csrc/fwd_order.hip",
            "block_sparse_cross_amd/csrc/fwd_common.h", "block_sparse_cross_amd/csrc/mfma_common.h"],
    "bwd": ["block_sparse_cross_amd/csrc/bwd_bf16.hip", "block_sparse_cross_amd/csrc/fwd_common.h",
            "block_sparse_cross_amd/csrc/mfma_common.h"],
}
INTERNAL_HEADER = "block_sparse_cross_amd/csrc/bsx_internal.h"


def sources_sha256(call: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in CALL_SOURCES[call]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    with open(os.path.join(ROOT, INTERNAL_HEADER), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def recorded_traffic(call: str, workload: str):
    """HBM bytes per call from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE of the call's kernels, scaled by the elementwise-kernel
    calibration), or None when there is none for this workload or the kernel sources
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{call}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic_record: "):
                rec = json.loads(line[len("traffic_record: "):])
                if rec.get("sources_sha256") == sources_sha256(call):
                    return rec["bytes_per_launch"]
    return None


def context_sweep(device, steps: int = 20, warmup: int = 3):
    """Fixed query budget (512 draft queries), context S = 16K .. 1M: useful TFLOP/s of the
    step and of the forward launch, per S."""
    import torch

    from workloads import SWEEP_CTX, make_workload, sweep_config

    rows = []
    for S in SWEEP_CTX:
        wl = make_workload(sweep_config(S))
        st = Step(wl, device, device_kv=True)
        st.prepare()
        for _ in range(warmup):
            st.run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.run()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        fwd_s = time_forward(st, 10)
        rows.append({"ctx_len": S, "n_queries": wl.n_queries, "ms_per_step": round(dt * 1e3, 4),
                     "step_tflops": round(st.step_flops / dt / 1e12, 2),
                     "fwd_us": round(fwd_s * 1e6, 2),
                     "fwd_tflops": round(st.fwd_flops / fwd_s / 1e12, 2),
                     "lpt_imbalance": round(st.plan0.imbalance, 5)})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
        del st
        torch.cuda.empty_cache()
    return rows


def cost_stress(device, reps: int = 20):
    """Cost kernel at a write-bound size: 65536 draft blocks x 4096 chunks of 1024 keys
    (2 GiB of int64 counts).  Algorithmic bytes: block ranges and chunk table read,
    counts and chunk costs written."""
    import torch

    import block_sparse_cross_amd as bsx

    nb, nc, L = 65536, 4096, 1024
    S = nc * L
    rng = np.random.default_rng(23)
    anchor = rng.integers(0, S + 1, size=nb)
    begin = np.minimum(anchor, rng.integers(0, S + 1, size=nb))
    shape = bsx.Shape(n_blocks=nb, block_size=16, n_q_heads=32, n_kv_heads=4, ctx_len=S)
    chunks = bsx.Chunks(np.arange(nc) * L, np.full(nc, L))
    an = torch.from_numpy(anchor).to(device)
    be = torch.from_numpy(begin).to(device)
    counts = torch.empty((nb, nc), dtype=torch.int64, device=device)
    cost = torch.empty(nc, dtype=torch.int64, device=device)
    err = torch.empty(1, dtype=torch.int32, device=device)
    ws = torch.empty(max(bsx.cost_workspace_bytes(nc), 256), dtype=torch.uint8, device=device)
    call = bsx.prepare_cost(shape, an, be, chunks, cost, err, counts=counts, ws=ws)
    for _ in range(3):
        call()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    e1.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    nbytes = 16 * nb + 16 * nc + 8 * nb * nc + 8 * nc + 4
    return {"n_blocks": nb, "n_chunks": nc, "chunk_len": L, "launch_us": round(us, 2),
            "bytes_per_launch": nbytes, "achieved_GBs": round(nbytes / us / 1e3, 1),
            "peak_GBs": PEAK_HBM_GBS, "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
            "mask_err": int(err.item())}


def planner_comparison(device, reps: int = 2000):
    """Chunk placements on the planned workloads' realized costs (cost kernel on the GPU):
    imbalance and host time per plan for LPT and the static layouts the pages compare.
    Host time is the C call alone: the library entry point is called through ctypes with
    its arguments marshalled once, and the same loop around a call that returns at once
    (bsx_abi_version) is subtracted."""
    import ctypes

    import torch

    import block_sparse_cross_amd as bsx
    from block_sparse_cross_amd._lib import lib
    from workloads import get_config, make_workload

    L = lib()

    def loop_ns(fn, args):
        t0 = time.perf_counter_ns()
        for _ in range(reps):
            fn(*args)
        return (time.perf_counter_ns() - t0) / reps

    base = min(loop_ns(L.bsx_abi_version, ()) for _ in range(5))
    out = {}
    for name in ("b27_s64k", "rank_p64_s1m", "train_pack128k"):
        cfg = get_config(name)
        wl = make_workload(cfg)
        shape = bsx.Shape(wl.n_blocks, cfg.block_size, cfg.n_q_heads, cfg.n_kv_heads, cfg.ctx_len)
        an = torch.from_numpy(wl.anchor).to(device)
        be = torch.from_numpy(wl.ctx_begin).to(device)
        _, cost, _ = bsx.cost(shape, an, be, bsx.Chunks(wl.chunk_start, wl.chunk_len),
                              with_counts=False)
        cost = np.ascontiguousarray(cost.cpu().numpy(), np.int64)
        n, P = int(cost.shape[0]), int(cfg.n_bins)
        bin_of = np.empty(n, np.int32)
        loads = np.empty(P, np.int64)
        ms, imb = ctypes.c_int64(0), ctypes.c_double(0.0)
        res = {"n_chunks": n, "n_bins": P}
        for mode in ("lpt", "zigzag", "round_robin", "contiguous"):
            r = bsx.place(mode, cost, P)
            args = (bsx.api.PLACEMENTS[mode], n, cost.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                    P, bin_of.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                    loads.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), ctypes.byref(ms),
                    ctypes.byref(imb))
            ns = min(loop_ns(L.bsx_place, args) for _ in range(5))
            res[mode] = {"imbalance": round(r.imbalance, 5), "ns_per_call": round(ns, 1),
                         "ns_net_of_call_overhead": round(ns - base, 1)}
        out[name] = res
    out["call_overhead_ns"] = round(base, 1)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU Split-KV exchange is not implemented here)", file=sys.stderr)
        sys.exit(2)
    import torch

    from workloads import get_config, make_workload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        print(json.dumps({"sweep": context_sweep(dev)}), flush=True)
        return
    if args.cost_stress:
        print(json.dumps({"cost_stress": cost_stress(dev)}), flush=True)
        return
    if args.planners:
        print(json.dumps({"planners": planner_comparison(dev),
                          "note": "ns_per_call: the C entry point through ctypes with "
                                  "pre-marshalled arguments; net: minus an empty call"}),
              flush=True)
        return
    if args.calibrate_copy_mib > 0:
        # a plain elementwise kernel of known traffic (reads and writes N MiB with
        # ordinary loads and stores), the reference for the HBM byte counters
        n = args.calibrate_copy_mib << 18  # float32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    cfg = get_config(args.workload)
    wl = make_workload(cfg, args.seed)
    # sweep workloads draw their (large) context K/V on the device: timing only
    step = Step(wl, dev, device_kv=cfg.name.startswith("sweep_"))
    step.prepare()
    print(f"# workload {cfg.name}: blocks={wl.n_blocks} queries={wl.n_queries} "
          f"local_chunks={len(step.plan0.local_chunks)} fwd useful GFLOP={step.fwd_flops / 1e9:.2f}",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step.run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt / args.steps * 1e3
    value = step.step_flops / (dt / args.steps) / 1e12

    # the dominant call of the step (the backward on the training workload) gives the
    # roofline; the forward call's roofline is reported beside it
    fwd_rl = fwd_roofline(step, args.fwd_reps, cfg.name)
    roofline = fwd_rl
    bwd_rl = None
    if step.bwd_call is not None:
        bwd_rl = bwd_roofline(step, args.fwd_reps, cfg.name)
        if bwd_rl["launch_us"] > fwd_rl["launch_us"]:
            roofline = bwd_rl
    other_fwd = {}
    if not args.no_extra_fwd and cfg.dtype == "bf16":
        # the forward of the other two large workloads, in the launch configuration their
        # steps use (LPT-bin slots; one rank's fused share)
        for name in ("b27_s64k", "rank_p64_s1m"):
            if name == cfg.name:
                continue
            wl2 = make_workload(get_config(name))
            st2 = Step(wl2, dev)
            st2.prepare()
            other_fwd[name] = fwd_roofline(st2, args.fwd_reps, name)
            del st2
            torch.cuda.empty_cache()
    merge = None if args.no_merge_bench else merge_bench(dev)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(wl, step.plan0, args.cpu_seconds)

    c = cfg
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "dtype": c.dtype, "data": "synthetic",
        "config": {"workload": c.name, "ctx_len": c.ctx_len, "n_q_heads": c.n_q_heads,
                   "n_kv_heads": c.n_kv_heads, "head_dim": c.head_dim,
                   "n_anchors": wl.n_blocks, "block_size": c.block_size,
                   "n_queries": wl.n_queries, "chunk_len": c.chunk_len,
                   "n_chunks": wl.n_chunks, "slot_mode": c.slot_mode, "n_bins": c.n_bins,
                   "backward": c.backward, "seed": wl.cfg.seed},
        "roofline": roofline,
        "fwd_roofline": fwd_rl,
        "bwd_roofline": bwd_rl,
        "fwd_roofline_other_workloads": other_fwd or None,
        "merge_roofline": merge,
        "cpu_baseline": cpu,
    }
    if c.slot_mode != "per_chunk":
        line["lpt_imbalance"] = step.plan0.imbalance
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
