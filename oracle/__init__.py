"""CPU oracle for the ISA forward pass.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke entry point and the
benchmark's CPU-baseline leg, never by the HIP library or its Python binding.
It shares no code with the HIP path; both take their inputs from the seeded
generator module isa_inputs, which holds no arithmetic of the method.
"""
from .isa_oracle import (Plan, make_plan, pool, coarse_scores, context_scores, top_k,
                         sharpness, split, kept_blocks, exact_sets, isa_head, isa_forward,
                         dense_attention, HeadResult, coarse_output, rope, rope_positions,
                         rope_tables, isa_head_backward, isa_head_dq_rows, rope_backward)

__all__ = ["Plan", "make_plan", "pool", "coarse_scores", "context_scores", "top_k",
           "sharpness", "split", "kept_blocks", "exact_sets", "isa_head", "isa_forward",
           "dense_attention", "HeadResult", "coarse_output", "rope", "rope_positions",
           "rope_tables", "isa_head_backward", "isa_head_dq_rows", "rope_backward"]
