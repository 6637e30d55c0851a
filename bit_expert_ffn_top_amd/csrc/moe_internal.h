// Host-side launchers shared between the translation units of the library.
// Every launcher assumes its arguments were validated by the C ABI layer and
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitffn_moe.h"
#include "moe_common.h"

namespace bitffn {

// Router projection, T <= MOE_MAX_DECODE_T tokens (router.hip).
hipError_t launch_router_logits(const float* x, int T, int d, const uint16_t* w, int E,
                                float* logits, hipStream_t s);

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx,
                             float* w, hipStream_t s);

hipError_t launch_lookup_slots(const int32_t* idx, int T, int k, const int32_t* table,
                               int32_t* slot, hipStream_t s);

// Small lookup: one workgroup, T*k <= kSmallLookupPairs.
constexpr int kSmallLookupPairs = 1024;
hipError_t launch_lookup_small(const int32_t* idx, int T, int k, const int32_t* table, int E,
                               int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                               int32_t* n_miss, hipStream_t s);

// Grouping of (t, i) pairs by expert id, stable in (t, i) order, for the pairs
// whose slot satisfies the predicate (hits: 0 <= slot < n_slots, misses:
// slot < 0; n_slots is read only for hits).
// Outputs: offsets[E+1] (may be null), perm (pair ids in group order),
// pos[T*k] (position of each pair, -1 if not selected; may be null),
// distinct[E] (ascending ids of non-empty groups; may be null),
// counts_out[2] = {non-empty groups, selected pairs} (may be null),
// tile_base[E+2] (may be null): prefix sums of ceil(group size / tile_m) for
// the E groups plus one extra group of T rows (the shared expert);
// tile_group[tile_base[E+1]] (may be null, needs tile_base): the group of
// every tile; group_slot[E] (may be null): the slot of the first selected
// pair of every non-empty group (all its pairs name one expert, so one slot).
struct GroupWorkspace {
  int32_t* chunk_counts;  // [n_chunks * E]
  int32_t* totals;        // [2 * MOE_MAX_EXPERTS]: per-expert totals, then group starts
};
constexpr int kGroupChunkTokens = 32;
size_t group_workspace_bytes(int T, int E);
GroupWorkspace group_workspace(void* ws, int T, int E);
hipError_t launch_group_pairs(const int32_t* idx, const int32_t* slot_of_pair,
                              const int32_t* table, int T, int k, int E, bool select_hits,
                              int n_slots, GroupWorkspace gws, int32_t* offsets, int32_t* perm,
                              int32_t* pos, int32_t* distinct, int32_t* counts_out,
                              int32_t* tile_base, int tile_m, int32_t* tile_group,
                              int32_t* group_slot, hipStream_t s);

// Compute units of the current device (looked up once per device).
constexpr int kMaxDevices = 64;
int device_cus();

size_t decode_workspace_bytes(int d, int f, int T, int k);
hipError_t launch_decode(const moe_layer& L, const float* x, int T, const int32_t* idx,
                         const int32_t* slot, const float* w, float* y, void* ws,
                         hipStream_t s);

// Route, look up and run the decode layer in two launches (routing runs in
// every FFN workgroup; workgroup (0, 0) writes the routing outputs).  y may be
// null if xnext is given; xnext (optional) receives y + addend (addend
// optional), the next layer's input in a decode step.
hipError_t launch_decode_layer(const moe_layer& L, const float* x, int T, const float* logits,
                               const int32_t* slot_of_expert, int32_t* idx, float* w,
                               int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                               int32_t* n_miss, float* y, void* ws, hipStream_t s,
                               float* xnext = nullptr, const float* addend = nullptr);
// The decode layer with the misses read from a second pool (host tier) in the
// same launch as the hits (moe_decode_layer_tiers).
hipError_t launch_decode_layer_tiers(const moe_layer& L, const moe_layer& H,
                                     const void* host_pool_dev, const int32_t* host_slot_of_expert,
                                     int max_rank, const float* x, int T, const float* logits,
                                     const int32_t* slot_of_expert, int32_t* idx, float* w,
                                     int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                                     int32_t* n_miss, float* y, void* ws, hipStream_t s);

// Missed pairs of a decode step computed from a second pool (the host tier,
// `host_pool_dev` its device-side address) and added into y; `phases` selects
// the read (their products into the workspace) and the join (y += them).
hipError_t launch_decode_misses(const moe_layer& H, const void* host_pool_dev, const float* x,
                                int T, const int32_t* idx, const int32_t* slot, const float* w,
                                const int32_t* host_slot_of_expert, int max_rank, float* y,
                                void* ws, hipStream_t s, int phases = MOE_MISSES_READ | MOE_MISSES_JOIN);

// Expert-cache admission and eviction (cache_policy.hip).
hipError_t launch_cache_count(const int32_t* idx, int n, int E, uint32_t* counts,
                              hipStream_t s);
hipError_t launch_cache_plan(uint32_t* counts, int E, int32_t* slot_of_expert,
                             int32_t* expert_of_slot, int n_slots, int shared_slot,
                             const int32_t* host_slot, int host_n_slots, int max_swaps,
                             int decay_shift, int32_t* swaps, int32_t* n_swaps, hipStream_t s);
hipError_t launch_cache_fill(const void* host_pool_dev, int host_n_slots, void* pool,
                             int n_slots, int64_t slot_bytes, const int32_t* swaps,
                             const int32_t* n_swaps, int max_swaps, hipStream_t s);
hipError_t launch_cache_commit(int32_t* slot_of_expert, int E, const int32_t* swaps,
                               const int32_t* n_swaps, int max_swaps, hipStream_t s);

// Copies of a whole layer into a staging pool in expert order (stage.hip).
// slot_of_expert and host_slot_of_expert are host arrays; every expert has a
// source (checked by the caller).
hipError_t launch_stage_layer(const moe_layer& C, const int32_t* slot_of_expert,
                              const void* host_pool, const int32_t* host_slot_of_expert,
                              void* staging, hipStream_t s);

// Decode through a stack of layers, one moe_decode_layer step per layer whose
// combine also forms the next layer's input (decode_stack.hip).
struct StackDims {
  int d, f, E, k, T;
};
size_t decode_stack_workspace_bytes(int d, int f, int T, int k);
hipError_t launch_decode_stack(const StackDims& D, int n_layers, const moe_stack_layer* layers,
                               const float* x, void* ws, hipStream_t s);

size_t prefill_workspace_bytes(int d, int f, int T, int k, int E);
hipError_t launch_prefill(const moe_layer& L, const uint16_t* x_bf16, int T,
                          const int32_t* idx, const int32_t* slot, float* out_pairs,
                          int32_t* pair_pos, int32_t* expert_offsets, float* out_shared,
                          void* ws, hipStream_t s);

hipError_t launch_combine(const void* x, int x_dtype, int T, int d, int k, const float* rows,
                          const int32_t* pair_pos, const float* w, const float* shared,
                          float* y, hipStream_t s);

}  // namespace bitffn
