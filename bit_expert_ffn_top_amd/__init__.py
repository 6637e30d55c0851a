"""MI355X (gfx950) routed-expert MoE layer over 2-3-bit block-quantized experts.

The computation lives in libbitffn_moe.so (HIP kernels behind the C ABI of
include/bitffn_moe.h); this package is its thin Python binding.
"""
from ._binding import (  # noqa: F401
    DTYPE_BF16, MISSES_JOIN, MISSES_READ, DTYPE_F32, FMT_Q2S, FMT_Q2SM, FMT_Q3G, HostTier, MoeError, MoeLayer,
    abi_version,
    cache_commit, cache_count, cache_fill, cache_lookup, cache_plan, combine,
    decode_layer, decode_layer_noalloc, decode_layer_tiers, decode_misses, decode_stack, decode_stack_workspace_bytes,
    decode_workspace_bytes, expert_ffn_decode, new_stack_workspace,
    expert_ffn_prefill, lib, lib_path, lookup_workspace_bytes, prefill_workspace_bytes,
    route_topk, router_logits, slot_bytes, stage_layer,
)
