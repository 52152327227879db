"""CPU oracle of the 4-bit grouped MoE layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package.  Parity status of each function is stated in its
docstring and in the pins under tests/ (test_oracle_*.py).
"""
from .moe_oracle import (  # noqa: F401
    bf16_bits_to_f64, f32_to_bf16_rne_bits, unpack_codes, dequant_bf16_bits, dequant,
    route_topk, max_blocks, group, silu, swiglu_ffn, moe_layer, moe_layer_chunked,
    router_logits, shared_gate,
)
