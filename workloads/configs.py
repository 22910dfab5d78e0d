"""Workload shapes for draft-query block-sparse cross-attention.

Head counts and head_dim follow the target-model shape table of the Split-KV
page ("Split-KV: Efficient Context Parallelism for Training Diffusion
Drafters", Figures & tables, target-model rows: 32 query heads, 4 or 8 KV
heads, head dim 128).  Context lengths, anchor counts, chunking, planner bin
counts and value scales are the five workload descriptions this library is
measured on; each field below states one of them.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    seed: int
    ctx_len: int            # S: packed context length (keys)
    n_q_heads: int          # H_q
    n_kv_heads: int         # H_kv
    head_dim: int           # d
    dtype: str              # "f32" or "bf16": the dtype of Q/K/V (and dO)
    sigma: float            # Q/K/V ~ N(0, 1) * sigma
    block_size: int         # B: draft queries per anchor block
    chunk_len: int          # every KV chunk has this many keys
    # single-sample anchor rule: n_anchors drawn without replacement from [anchor_lo, anchor_hi)
    n_anchors: int = 0
    anchor_lo: int = 0
    anchor_hi: int = 0
    # packed multi-sample rule (training step): n_samples lengths log-uniform in
    # [len_lo, len_hi], packed into ctx_len; floor(L_i / anchor_every) anchors per sample
    n_samples: int = 1
    len_lo: int = 0
    len_hi: int = 0
    anchor_every: int = 0
    # how chunks map to output slots of the forward pass
    slot_mode: str = "per_chunk"    # "per_chunk" | "lpt" | "rank"
    n_bins: int = 0                 # LPT bins (virtual context-parallel ranks)
    self_slot: bool = True          # the draft block's own keys form one more slot
    backward: bool = False
    # standalone merge of seeded partial sets (one rank's view at CP size n_merge_sets)
    n_merge_sets: int = 0
    merge_lse_shift: float = 0.0

    @property
    def n_chunks(self) -> int:
        return self.ctx_len // self.chunk_len

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def packed(self) -> bool:
        return self.n_samples > 1


CONFIGS = [
    # Tiny fp32 check: 1 sample, S=1024, GQA 8:2, 4 anchors in [64, 1024), 4 chunks of 256,
    # per-chunk partials + self slot, merged and compared with unchunked attention.
    WorkloadConfig(
        name="tiny_f32", seed=1, ctx_len=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
        dtype="f32", sigma=1.0, block_size=16, chunk_len=256,
        n_anchors=4, anchor_lo=64, anchor_hi=1024, slot_mode="per_chunk"),
    # Qwen3.5-35B-A3B drafter shape: S=16384, H_q=32, H_kv=4, 32 anchors in [256, 16384),
    # 16 chunks of 1024, per-chunk fp32 partials then merge.
    WorkloadConfig(
        name="a3b_s16k", seed=2, ctx_len=16384, n_q_heads=32, n_kv_heads=4, head_dim=128,
        dtype="bf16", sigma=0.5, block_size=16, chunk_len=1024,
        n_anchors=32, anchor_lo=256, anchor_hi=16384, slot_mode="per_chunk"),
    # Qwen3.5-27B drafter shape: S=65536, H_q=32, H_kv=8, 64 anchors in [512, 65536),
    # 64 chunks of 1024, cost -> LPT over 8 bins -> one partial per bin -> merge.
    WorkloadConfig(
        name="b27_s64k", seed=3, ctx_len=65536, n_q_heads=32, n_kv_heads=8, head_dim=128,
        dtype="bf16", sigma=0.5, block_size=16, chunk_len=1024,
        n_anchors=64, anchor_lo=512, anchor_hi=65536, slot_mode="lpt", n_bins=8),
    # One context-parallel rank at P=64: S=1M in 256 chunks of 4096, 128 anchors over the
    # whole context, LPT over 64 bins, attention over the most loaded bin's chunks into one
    # fused partial (no self slot); plus a standalone merge of 64 seeded partial sets.
    WorkloadConfig(
        name="rank_p64_s1m", seed=4, ctx_len=1 << 20, n_q_heads=32, n_kv_heads=4, head_dim=128,
        dtype="bf16", sigma=0.5, block_size=16, chunk_len=4096,
        n_anchors=128, anchor_lo=0, anchor_hi=1 << 20, slot_mode="rank", n_bins=64,
        self_slot=False, n_merge_sets=64, merge_lse_shift=8.0),
    # Training step: 8 samples, lengths log-uniform in [2048, 32768] packed into 131072,
    # one anchor per 1024 tokens of a sample, 128 chunks of 1024, LPT over 16 bins,
    # forward partials + merge, then dQ/dK/dV from seeded dO.
    WorkloadConfig(
        name="train_pack128k", seed=5, ctx_len=131072, n_q_heads=32, n_kv_heads=8,
        head_dim=128, dtype="bf16", sigma=0.5, block_size=16, chunk_len=1024,
        n_samples=8, len_lo=2048, len_hi=32768, anchor_every=1024,
        slot_mode="lpt", n_bins=16, backward=True),
]


# Fixed query budget, growing context (the query-context asymmetry the Split-KV page's
# Abstract describes: acceptance stays stable as the context grows at a fixed query
# budget): the a3b head shape with 32 anchors (512 draft queries) over S keys, chunks of
# 1024 balanced by LPT over 16 bins.
SWEEP_CTX = [16384, 32768, 65536, 131072, 262144, 524288, 1048576]


def sweep_config(ctx_len: int) -> WorkloadConfig:
    return WorkloadConfig(
        name=f"sweep_s{ctx_len}", seed=6, ctx_len=ctx_len, n_q_heads=32, n_kv_heads=4,
        head_dim=128, dtype="bf16", sigma=0.5, block_size=16, chunk_len=1024,
        n_anchors=32, anchor_lo=256, anchor_hi=ctx_len, slot_mode="lpt", n_bins=16)


def get_config(name_or_index) -> WorkloadConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    for c in CONFIGS:
        if c.name == name_or_index:
            return c
    if isinstance(name_or_index, str) and name_or_index.startswith("sweep_s"):
        return sweep_config(int(name_or_index[len("sweep_s"):]))
    raise KeyError(name_or_index)


def scaled_down(cfg: WorkloadConfig, **overrides) -> WorkloadConfig:
    """A copy of ``cfg`` with some fields replaced (for parity cases the oracle finishes fast)."""
    from dataclasses import replace
    return replace(cfg, **overrides)


def find(name: str) -> Optional[WorkloadConfig]:
    try:
        return get_config(name)
    except KeyError:
        return None
