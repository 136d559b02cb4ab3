"""CPU oracle of the MoE routing-and-combine path.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only tests/, the smoke check of
__graft_entry__ and the CPU-baseline leg of bench.py may import it. It shares
no code with the HIP library (moe_token_routing_amd) and neither imports the
other.

A plain, slow, obviously correct numpy implementation: float64 wherever the
method is a real-number formula, IEEE binary32 wherever the method fixes FP32
steps, no blocking, fusion or reordering beyond what each definition states.
Each function names the passage it follows.

Pins (tests/test_oracle_*.py, run without a GPU): brute force on tiny inputs,
closed forms (one-hot projections, power-of-two rows, sigmoid(0) = 1/2),
invariants (weights sum to 1, histogram sums to valid tokens x k, the
permutation is a bijection), exhaustive format tables and the thresholds the
quantizer page prints (tests/golden/).
"""
from .formats import (bf16_bits_to_f64, round_bf16, f64_to_bf16_bits, bf16_ulp,
                      e4m3_encode_satfinite, e4m3_decode, e2m1_encode, e2m1_decode,
                      E4M3_VALUES, E2M1_VALUES)
from .route import (router_logits, sigmoid_f32, selection_keys, topk_sorted,
                    renormalized_weights, route_from_logits, route, key_gap_near_ties)
from .dispatch import dispatch
from .nvfp4 import (gain_f32, rmsnorm_exact, rmsnorm_bf16, nvfp4_quantize,
                    norm_quant_nvfp4, global_scale, midpoint_boundary_blocks, dequantize,
                    rank_block_rows, norm_quant_nvfp4_rank_block)
from .combine import combine
from .fc1 import (relu2, silu, swiglu, SILU_ARGMIN, fc1_exact, expert_fc1_nvfp4, fc1_boundary_blocks,
                  expert_fc1_swiglu_nvfp4, fc1_swiglu_boundary_blocks, swiglu_boundary_from_values)

__all__ = [n for n in dir() if not n.startswith("_")]
