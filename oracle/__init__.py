"""CPU oracle for the routed-expert FFN (test infrastructure only).

Plain, slow NumPy in float64.  Only the tests, the package's smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code with the HIP library or with the input generator; it reads
the packed slot bytes with its own unpacker.

Parity status of each function is stated in its docstring.
"""
from .moe import (  # noqa: F401
    FMT_Q2S, FMT_Q2SM, FMT_Q3G, plane_offsets, slot_size, unpack_matrix,
    unpack_expert, bf16_bits_to_f64, router_logits, route_topk, cache_lookup, silu, expert_ffn, layer_decode, layer_decode_tiers,
    layer_dense_mixture, bf16_round, expert_ffn_bf16, permute_pairs, cache_count, cache_plan,
    cache_commit,
    prefill_layer, combine, union_plan,
)
