"""Seeded synthetic inputs for the speculative-decoding verify step.

This module is the single source of inputs shared by the CPU oracle and the
GPU library: model shapes, random-init weights, prompts, draft chains, draft
trees and the batched request mix.  It holds none of the model's arithmetic:
it draws numbers and shapes only.  Weights are plain N(0, 0.02) samples
(rounded to bf16 for the bf16 models): random-init models of the same
shapes stand in for the trained Qwen-family targets the pages evaluate
(SpecPilot paper card, abstract; besthub.dev article, "Experimental
Results").
"""

from .configs import MODELS, WORKLOADS, model_config, workload
from .weights import tensor_specs, make_weights, bf16_bits_to_f32
from .drafts import (prompt_tokens, chain_drafts, tree_topology, tree_drafts,
                     batched_mix, expected_tokens_per_step)

__all__ = [
    "MODELS", "WORKLOADS", "model_config", "workload",
    "tensor_specs", "make_weights", "bf16_bits_to_f32",
    "prompt_tokens", "chain_drafts", "tree_topology", "tree_drafts",
    "batched_mix", "expected_tokens_per_step",
]
