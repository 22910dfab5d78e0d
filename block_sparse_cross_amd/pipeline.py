"""One pass of the Split-KV hot path on one GPU, composed from the C ABI calls.

Split-KV page, Abstract: KV chunks stay local, their realized attention cost
feeds a longest-processing-time-first plan, every rank attends the full (global)
query set against its local chunks, and query-sized partials merge exactly.  On
one GPU the steps are:

  cost kernel  -> chunk costs (device; the one readback of the pass)
  LPT (host)   -> chunk -> slot map (per chunk, per virtual rank, or one rank's share)
  attention    -> per-slot partial (O, LSE) (device)
  LSE merge    -> merged (O, LSE) (device)
  backward     -> dQ, dK, dV (device; training only)

Slot modes: "per_chunk" (one partial per chunk), "lpt" (one partial per LPT bin,
i.e. per virtual context-parallel rank), "rank" (the most loaded bin's chunks only,
lowest bin index on ties, fused into one partial: one rank's share).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import api
from .api import Chunks, Shape


class MaskError(ValueError):
    """The cost kernel flagged a block range outside the context."""


@dataclass
class Plan:
    chunk_cost: np.ndarray          # int64 [n_chunks], from the cost kernel
    bin_of: Optional[np.ndarray]    # int32 [n_chunks] LPT bin per chunk (lpt/rank modes)
    loads: Optional[np.ndarray]
    makespan: int
    imbalance: float
    local_chunks: np.ndarray        # chunk ids held in the local K/V buffer, in buffer order
    chunks: Chunks                  # chunk table of the local buffer, with output slots
    rank: int = -1                  # the chosen bin in "rank" mode


def make_plan(shape: Shape, chunk_start, chunk_len, mode: str, n_bins: int,
              anchor: torch.Tensor, ctx_begin: torch.Tensor,
              cost_ws: Optional[torch.Tensor] = None, cost_out=None) -> Plan:
    all_chunks = Chunks(chunk_start, chunk_len)
    _, chunk_cost, mask_err = api.cost(shape, anchor, ctx_begin, all_chunks, with_counts=False,
                                       ws=cost_ws, out=cost_out)
    cost_host = chunk_cost.cpu().numpy()
    if int(mask_err.cpu().item()) != 0:
        raise MaskError("some draft block's context range [ctx_begin, anchor) is not an "
                        f"interval of [0, {shape.ctx_len}]: the plan would use clamped ranges")
    start = np.asarray(chunk_start, np.int64)
    length = np.asarray(chunk_len, np.int64)
    n = start.shape[0]
    if mode == "per_chunk":
        return Plan(cost_host, None, None, 0, 0.0, np.arange(n),
                    Chunks(start, length, None, n))
    r = api.lpt(cost_host, n_bins)
    if mode == "lpt":
        return Plan(cost_host, r.bin_of, r.loads, r.makespan, r.imbalance, np.arange(n),
                    Chunks(start, length, r.bin_of, n_bins))
    if mode == "rank":
        rank = int(np.argmax(r.loads))  # first index among the maxima
        mine = np.nonzero(r.bin_of == rank)[0]
        return Plan(cost_host, r.bin_of, r.loads, r.makespan, r.imbalance, mine,
                    Chunks(start[mine], length[mine], np.zeros(len(mine), np.int32), 1), rank)
    raise ValueError(f"unknown slot mode {mode!r}")
