"""CPU oracle for the speculative-decoding verify step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the GPU library.

What it computes is the plain definition of lossless greedy speculative
verification: a target model scores a root plus a tree (or chain) of draft
tokens in one pass, takes the greedy argmax at every node and accepts the
longest root path whose tokens match the target's own choices, so the emitted
text equals plain autoregressive greedy decoding ("token forcing" checks
exactly this; zicq.com article, "Core Idea: Let Agents Discover the
Bottlenecks"; besthub.dev article, "Phase 4: Final Validation").
"""

from .model import (Model, State, bf16_round, rmsnorm, silu, sigmoid,
                    rope_tables, apply_rope, masked_attention, tree_layout)
from .verify import (accept_path, ar_greedy, verify_single_pass,
                     verify_bruteforce, top2_margin)

__all__ = [
    "Model", "State", "bf16_round", "rmsnorm", "silu", "sigmoid",
    "rope_tables", "apply_rope", "masked_attention", "tree_layout",
    "accept_path", "ar_greedy", "verify_single_pass", "verify_bruteforce",
    "top2_margin",
]
