"""fp64 CPU oracle for dynamic top-k sparse attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the product path.
"""
from .sparse_attn_oracle import (  # noqa: F401
    f64, project, valid_keys, score_rows, scores, topk_row, topk_rows,
    topk_indices, brute_force_topk, attend_row, gather_attention,
    sparse_attn_fwd, band_indices, dense_attention, local_mask,
    brute_force_attention, attend_row_backward, sparse_attn_backward,
    smoothed_topk_row, smoothed_topk_rows, dilated_indices, band_indices_per_batch,
    decode_step, block_means, block_select_row, block_keys_row, block_topk_indices,
)
from .compare import row_invariants, set_overlap  # noqa: F401
