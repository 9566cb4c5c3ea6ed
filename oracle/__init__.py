"""CPU oracle of the routed MoE expert-FFN path (float64, numpy).

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it.  The GPU library never imports,
links or calls anything here, and nothing here is shared with it.

Parity status: every function is pinned by a CPU test (tests/test_oracle_*.py)
against something other than itself — torch's dtype tables, hand-worked
closed-form cases, a dense no-routing equivalence, an independent float64
matmul chain, brute-force routing/permutation invariants.  No function is
parity unpinned.
"""
from .codecs import (bf16_decode, e2m1_decode_nibbles, e2m1_unpack, e4m3_decode, round_bf16, round_e2m1_sat,
                     round_e4m3_sat, round_to_grid, ue8m0_decode)
from .moe import (BF16, FP8_BLOCK128, NVFP4, NVFP4_W4A16, W4A8_MX, Geometry, build_plan, combine, dequant_activations,
                  dequant_expert, dequant_fp8_block, dequant_mx, dequant_nvfp4, expert_rows, forward, forward_tokens,
                  mx_exponent, requant, requant_fp8_block128, requant_mx, requant_nvfp4, route_from_logits,
                  route_from_logits_fast, silu, swiglu_clamped)

__all__ = [
    "BF16", "FP8_BLOCK128", "NVFP4", "NVFP4_W4A16", "W4A8_MX", "Geometry", "bf16_decode", "build_plan", "combine",
    "dequant_activations", "dequant_expert", "dequant_fp8_block", "dequant_mx", "dequant_nvfp4", "e2m1_decode_nibbles",
    "e2m1_unpack", "e4m3_decode", "expert_rows", "forward", "forward_tokens", "mx_exponent", "requant",
    "requant_fp8_block128", "requant_mx", "requant_nvfp4", "round_bf16", "round_e2m1_sat", "round_e4m3_sat",
    "round_to_grid", "route_from_logits", "route_from_logits_fast", "silu", "swiglu_clamped", "ue8m0_decode",
]
