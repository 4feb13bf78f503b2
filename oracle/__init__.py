"""fp64 CPU oracle for Top-p block-sparse attention (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The GPU library never calls it, links it or falls back
to it, and it imports nothing from the GPU path.
"""
from .topp_oracle import (  # noqa: F401
    block_bounds, pool_blocks, block_scores, block_importance, routing_order,
    topp_count, route_head, route, sparse_attention_rows, sparse_attention,
    dense_attention, lpt_worklist, csr_rows, selection_count, window_blocks, sasa_augment,
    route_sasa, sasa_budget, unit_work, head_loads, lpt_units, heads_by_load, head_lpt_units,
    head_desc_units, rlb_assign, rlb_units,
)
