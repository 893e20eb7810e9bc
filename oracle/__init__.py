"""fp64 CPU oracle of the hybrid block-sparse attention path (test infrastructure
only: tests/, the smoke check and the benchmark's CPU-baseline leg use it; the
GPU package never does)."""
from .oracle import *  # noqa: F401,F403
from .oracle import (Geometry, MaskResult, RowSelection, attention_block,
                     block_scores, block_softmax, build_mask, ceil_k, coarse_output,
                     expand_blocks, pool_r, router_scores, subcube_of_slot,
                     sparse_attention_backward, pooled_mass, mask_error,
                     dense_attention, pool, rank_order, real_slots, reorder,
                     select_row, select_rows, sparse_attention, token_slots,
                     top_p_count, unreorder, unreorder_rows, NEAR_TIE,
                     group_count, pool_groups, build_mask_groups, expand_group_lists,
                     sequence_budget, per_sequence_counts, per_sequence_near_tie, build_mask_per_sequence,
                     ideal_block_mass, mask_recall, error_terms, mask_report)
