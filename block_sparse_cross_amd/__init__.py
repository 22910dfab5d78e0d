"""Block-sparse draft-query cross-attention on MI355X (gfx950).

The hot path of Split-KV context parallelism on one GPU ("Split-KV: Efficient
Context Parallelism for Training Diffusion Drafters", Abstract): a per-chunk
visible-key cost kernel feeding a longest-processing-time-first planner,
bf16 matrix-core attention kernels that emit per-slot partial outputs with their
log-sum-exp, an exact LSE merge, and the attention backward.

All computation lives in the HIP library ``libbsx.so`` (C ABI: ``include/bsx.h``);
this package only marshals torch tensors (device memory, current stream) into it.
"""
from .api import (BsxError, Chunks, LptResult, Prepared, Shape, abi_version,  # noqa: F401
                  attn_bwd, attn_fwd, bwd_workspace_bytes, cost, cost_workspace_bytes,
                  fwd_workspace_bytes, lpt, lse_merge, mask_from_anchors, place,
                  prepare_attn_bwd, prepare_attn_fwd, prepare_cost, prepare_lse_merge,
                  validate_mask)
from ._lib import lib as load_library  # noqa: F401
