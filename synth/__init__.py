"""Seeded synthetic inputs for tree verification.

This package builds the problem instances that both the CPU oracle and the HIP
path consume: draft trees (parent arrays, draft tokens), draft distributions q,
target logits, attention inputs and per-node uniforms.  It holds none of the
verification arithmetic itself: no tree mask, no attention, no target softmax,
no accept/reject rule.  The draft distribution q and the draft tokens are the
drafter's outputs, so producing them belongs here (a synthetic drafter).
"""
from .configs import CONFIGS, config_by_name, kv_head_shard, small_spec
from .gen import (Instance, make_instance, bf16_bits_from_f32, f32_from_bf16_bits,
                  tree_from_widths, random_tree_widths, make_draft_rows, make_head_inputs)

__all__ = ["CONFIGS", "config_by_name", "kv_head_shard", "small_spec", "Instance", "make_instance",
           "bf16_bits_from_f32", "f32_from_bf16_bits", "tree_from_widths",
           "random_tree_widths", "make_draft_rows", "make_head_inputs"]
