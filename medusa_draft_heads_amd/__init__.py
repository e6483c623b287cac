"""Medusa tree-decode step on AMD Instinct MI355X (gfx950).

The compute path is libmedusa (hand-written HIP kernels behind the C-ABI in
include/medusa.h); this package binds it with ctypes and drives a step.
PyTorch supplies device memory and streams only.
"""
from ._lib import (MD_BF16, MD_F32, MD_HEADS_HYDRA, MD_HEADS_MEDUSA, MD_HEADS_MEDUSA_SHARED, MedusaError, make_tree,
                   md_accept_workspace_bytes, md_attention_workspace_bytes, md_hbm_read_probe,
                   md_hbm_read_probe_blocks, md_heads_weight_bytes, md_heads_workspace_bytes, md_last_error,
                   md_medusa_heads, md_set_vocab_timing_events, md_target_argmax, md_target_argmax_workspace_bytes,
                   md_tree, md_tree_accept, md_tree_accept_tokens, md_tree_attention, md_tree_build, md_tree_validate,
                   md_heads_logits_workspace_bytes, md_medusa_heads_logits, md_draft_sample_workspace_bytes,
                   md_draft_sample, md_verify_sampled_workspace_bytes, md_tree_verify_sampled,
                   md_accept_typical_workspace_bytes, md_tree_accept_typical, md_operand_order_bytes,
                   md_operand_order, operand_order, md_certified_rounding_allowance, md_tree_attention_noalloc,
                   md_tree_attention_noalloc_max_bytes, md_heads_fused, md_set_wait_limits, md_vocab_tile_norms_bytes,
                   md_vocab_tile_norms, vocab_tile_norms)
from .step import MedusaStep, StepConfig

__all__ = [
    "MD_BF16", "MD_F32", "MD_HEADS_HYDRA", "MD_HEADS_MEDUSA", "MD_HEADS_MEDUSA_SHARED", "MedusaError", "make_tree", "md_tree",
    "md_medusa_heads", "md_tree_build", "md_tree_attention", "md_tree_accept", "md_tree_validate",
    "md_heads_weight_bytes", "md_heads_workspace_bytes", "md_attention_workspace_bytes", "md_accept_workspace_bytes",
    "md_set_vocab_timing_events", "md_last_error", "md_hbm_read_probe", "md_hbm_read_probe_blocks",
    "md_target_argmax", "md_target_argmax_workspace_bytes", "md_tree_accept_tokens",
    "md_heads_logits_workspace_bytes", "md_medusa_heads_logits", "md_draft_sample_workspace_bytes", "md_draft_sample",
    "md_verify_sampled_workspace_bytes", "md_tree_verify_sampled", "md_accept_typical_workspace_bytes",
    "md_tree_accept_typical", "md_operand_order_bytes", "md_operand_order", "operand_order",
    "md_certified_rounding_allowance", "md_tree_attention_noalloc", "md_tree_attention_noalloc_max_bytes",
    "md_heads_fused", "md_set_wait_limits", "md_vocab_tile_norms_bytes", "md_vocab_tile_norms", "vocab_tile_norms",
    "MedusaStep", "StepConfig",
]
