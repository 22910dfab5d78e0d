"""Seeded synthetic workloads for block-sparse draft-query cross-attention.

This package only *draws* inputs (anchor positions, sample lengths, Q/K/V
tensors, upstream gradients) and describes workload shapes.  It holds none of
the method's arithmetic: visibility, costs, plans, attention and merges are
computed separately by the fp64 oracle (``oracle/``) and by the HIP library
(``block_sparse_cross_amd``), which share nothing but these inputs.
"""
from .configs import CONFIGS, SWEEP_CTX, WorkloadConfig, get_config, sweep_config  # noqa: F401
from .gen import Workload, make_workload, draw_kv_chunks, draw_merge_sets  # noqa: F401
