"""fp64 CPU oracle for block-sparse draft-query cross-attention (Split-KV's local hot path).

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the CPU
baseline leg of the benchmark import this package.  The HIP library never calls
it, shares no code with it, and fails loudly instead of falling back to it.

Every function here is the plain definition, written in float64 on the exact
input values (bf16 inputs are upcast from their stored values), with a matmul,
exp, log, max or sum from NumPy as its only library steps.  Sources:

* "Split-KV: Efficient Context Parallelism for Training Diffusion Drafters",
  Abstract: draft queries built by anchor sampling cross-attend a much longer
  context under a block-sparse mask; the context-parallel method is exact, keeps
  key/value shards local, exchanges only query-sized tensors, and balances
  context KV chunks by their realized attention cost with longest-processing-
  time-first (LPT) planning.
* "Flash-dLLM: IO-Aware KV Caching and Parallel Decoding for Diffusion LLMs",
  section "Method 1: I/O-Aware Fused KV-Cache Kernel": attention is
  softmax(Q K^T / sqrt(d)) V.

Readings taken where the pages leave a step open are stated in each module.
Parity pins for every function live in ``tests/test_oracle_*.py``.
"""
from .mask import visible_context, mask_error  # noqa: F401
from .attention import (  # noqa: F401
    partial_attention, attention_block, attention, slot_partial_block, slot_partials,
    chunk_offsets, default_scale)
from .merge import lse_merge  # noqa: F401
from .cost import chunk_costs  # noqa: F401
from .lpt import lpt, lpt_makespan_opt  # noqa: F401
from .placement import contiguous, zigzag, round_robin  # noqa: F401
from .backward import attention_backward  # noqa: F401
