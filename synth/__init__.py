"""Seeded synthetic inputs for the routed-expert FFN.

This package makes inputs only: expert weights drawn from a normal law and
block-quantized into packed slot bytes, activations, router logits, slot
tables.  It holds none of the layer's arithmetic (no dequantization, no
routing, no FFN); the oracle and the HIP path each do that on their own.
"""
from .gen import (  # noqa: F401
    BASE_SEED, WORKLOADS, FMT_Q2S, FMT_Q2SM, FMT_Q3G, LayerShape,
    seed_of, torch_gen, slot_layout, slot_bytes, quantize_blocks,
    pack_matrix_planes, pack_expert_slots, expert_weights, make_layer_pool,
    make_x, make_logits, make_router_weights, make_slot_table, zipf_gumbel_logits, zipf_residency, zipf_popularity,
    config_shape, layer_format,
)
