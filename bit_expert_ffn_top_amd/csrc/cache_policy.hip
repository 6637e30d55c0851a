// Expert-cache admission and eviction: usage counts, a planned set of swaps,
// the copy of the admitted experts' bytes into their slots, and the commit
// that makes them visible in the slot table.
//
// Plan (one workgroup, n_experts <= 1024 so one expert per thread):
//   candidates  experts not resident, with a host copy and a count above 0,
//               ranked best first by (count desc, id asc);
//   victims     the cache's slots except the shared expert's, ranked worst
//               first by (count of the expert held asc, empty slots first,
//               slot asc);
//   the i-th candidate replaces the i-th victim while i < max_swaps and its
//   count is strictly above the victim's.  Both rankings come from counting,
//   for each key, how many keys beat it (LDS broadcast reads), so the result
//   is unique and independent of timing.
// The candidate ordering is monotone and the victim ordering too, so the
// swaps taken form a prefix of the rank order.
#include "moe_internal.h"

namespace bitffn {
namespace {

constexpr int kPlanThreads = 1024;
static_assert(MOE_MAX_EXPERTS <= kPlanThreads, "one expert per plan thread");

__global__ void cache_count_kernel(const int32_t* __restrict__ idx, int n, int E,
                                   uint32_t* __restrict__ counts) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= n) return;
  const int e = idx[p];
  if (e >= 0 && e < E) atomicAdd(counts + e, 1u);
}

__global__ __launch_bounds__(kPlanThreads) void cache_plan_kernel(
    uint32_t* __restrict__ counts, int E, int32_t* __restrict__ slot_of_expert,
    int32_t* __restrict__ expert_of_slot, int n_slots, int shared_slot,
    const int32_t* __restrict__ host_slot, int host_n_slots, int max_swaps, int decay_shift,
    int32_t* __restrict__ swaps, int32_t* __restrict__ n_swaps) {
  __shared__ uint32_t s_cnt[MOE_MAX_EXPERTS];
  __shared__ uint64_t s_ck[MOE_MAX_EXPERTS];     // candidate key, 0: not a candidate
  __shared__ uint64_t s_vk[MOE_MAX_CACHE_SLOTS];  // victim key, ~0: not a victim
  __shared__ int32_t s_cand_at[MOE_MAX_EXPERTS];  // candidate of rank i
  __shared__ int32_t s_vict_at[MOE_MAX_EXPERTS];  // victim slot of rank i
  const int tid = threadIdx.x;

  // counts and candidate keys: larger key = better candidate
  if (tid < E) {
    const uint32_t c = counts[tid];
    const int h = host_slot[tid];
    s_cnt[tid] = c;
    const bool cand = slot_of_expert[tid] < 0 && h >= 0 && h < host_n_slots && c > 0;
    s_ck[tid] = cand ? (static_cast<uint64_t>(c) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(tid))
                     : 0ull;
  }
  if (tid < max_swaps) {
    s_cand_at[tid] = -1;
    s_vict_at[tid] = -1;
  }
  __syncthreads();
  // victim keys: smaller key = evicted first; an empty slot (or one holding
  // an id outside [0, E)) has count -1, stored as 0 after the +1 offset
  for (int s = tid; s < n_slots; s += kPlanThreads) {
    if (s == shared_slot) {
      s_vk[s] = ~0ull;
      continue;
    }
    const int e = expert_of_slot[s];
    const uint64_t c1 = e >= 0 && e < E ? static_cast<uint64_t>(s_cnt[e]) + 1u : 0u;
    s_vk[s] = (c1 << 20) | static_cast<uint32_t>(s);
  }
  __syncthreads();

  // ranks by counting the keys that beat each one
  if (tid < E) {
    const uint64_t k = s_ck[tid];
    if (k != 0ull) {
      int r = 0;
      for (int j = 0; j < E; ++j) r += s_ck[j] > k ? 1 : 0;
      if (r < max_swaps) s_cand_at[r] = tid;
    }
  }
  for (int s = tid; s < n_slots; s += kPlanThreads) {
    const uint64_t k = s_vk[s];
    if (k != ~0ull) {
      int r = 0;
      for (int j = 0; j < n_slots; ++j) r += s_vk[j] < k ? 1 : 0;
      if (r < max_swaps) s_vict_at[r] = s;
    }
  }
  __syncthreads();

  // swap i happens if both ranks exist and the candidate's count is strictly
  // above the victim's (a prefix of i)
  int e = -1, s = -1, go = 0;
  if (tid < max_swaps) {
    e = s_cand_at[tid];
    s = s_vict_at[tid];
    if (e >= 0 && s >= 0)
      go = static_cast<int64_t>(s_cnt[e]) > static_cast<int64_t>(s_vk[s] >> 20) - 1 ? 1 : 0;
  }
  const int n = __syncthreads_count(go);
  if (go) {
    const int held = expert_of_slot[s];
    const int old = held >= 0 && held < E ? held : -1;
    swaps[4 * tid + 0] = s;
    swaps[4 * tid + 1] = old;
    swaps[4 * tid + 2] = e;
    swaps[4 * tid + 3] = host_slot[e];
    if (old >= 0) slot_of_expert[old] = -1;   // leaves the cache now
    expert_of_slot[s] = e;                      // reserved for the newcomer
  }
  if (tid == 0) n_swaps[0] = n;
  if (tid < E) counts[tid] = s_cnt[tid] >> decay_shift;
}

// Copy of each admitted expert's slot bytes from the host tier: workgroup
// (chunk c, swap i).  Every lane moves 16-byte words; each thread first
// requests all its words of the chunk, then stores them.
constexpr int kFillThreads = 256;
constexpr int kFillChunks = 32;
constexpr int kFillWords = 16;   // words per thread per round

__global__ __launch_bounds__(kFillThreads) void cache_fill_kernel(
    const uint8_t* __restrict__ host_pool, int host_n_slots, uint8_t* __restrict__ pool,
    int n_slots, int64_t slot_bytes, const int32_t* __restrict__ swaps,
    const int32_t* __restrict__ n_swaps) {
  const int i = blockIdx.y;
  if (i >= n_swaps[0]) return;
  const int s = swaps[4 * i + 0];
  const int h = swaps[4 * i + 3];
  if (s < 0 || s >= n_slots || h < 0 || h >= host_n_slots) return;
  const int64_t words = slot_bytes / 16;
  const int64_t lo = words * blockIdx.x / kFillChunks, hi = words * (blockIdx.x + 1) / kFillChunks;
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(host_pool + h * slot_bytes);
  uint4* __restrict__ dst = reinterpret_cast<uint4*>(pool + s * slot_bytes);
  for (int64_t q0 = lo + threadIdx.x; q0 < hi; q0 += kFillThreads * kFillWords) {
    uint4 v[kFillWords];
#pragma unroll
    for (int j = 0; j < kFillWords; ++j) {
      const int64_t q = q0 + static_cast<int64_t>(j) * kFillThreads;
      v[j] = src[q < hi ? q : lo];
    }
#pragma unroll
    for (int j = 0; j < kFillWords; ++j) {
      const int64_t q = q0 + static_cast<int64_t>(j) * kFillThreads;
      if (q < hi) dst[q] = v[j];
    }
  }
}

__global__ void cache_commit_kernel(int32_t* __restrict__ slot_of_expert, int E,
                                    const int32_t* __restrict__ swaps,
                                    const int32_t* __restrict__ n_swaps, int max_swaps) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= min(n_swaps[0], max_swaps)) return;
  const int e = swaps[4 * i + 2];
  if (e >= 0 && e < E) slot_of_expert[e] = swaps[4 * i + 0];
}

}  // namespace

hipError_t launch_cache_count(const int32_t* idx, int n, int E, uint32_t* counts,
                              hipStream_t s) {
  if (n == 0) return hipSuccess;
  cache_count_kernel<<<(n + 255) / 256, 256, 0, s>>>(idx, n, E, counts);
  return hipGetLastError();
}

hipError_t launch_cache_plan(uint32_t* counts, int E, int32_t* slot_of_expert,
                             int32_t* expert_of_slot, int n_slots, int shared_slot,
                             const int32_t* host_slot, int host_n_slots, int max_swaps,
                             int decay_shift, int32_t* swaps, int32_t* n_swaps, hipStream_t s) {
  cache_plan_kernel<<<1, kPlanThreads, 0, s>>>(counts, E, slot_of_expert, expert_of_slot,
                                               n_slots, shared_slot, host_slot, host_n_slots,
                                               max_swaps, decay_shift, swaps, n_swaps);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const void* host_pool_dev, int host_n_slots, void* pool,
                             int n_slots, int64_t slot_bytes, const int32_t* swaps,
                             const int32_t* n_swaps, int max_swaps, hipStream_t s) {
  const dim3 grid(kFillChunks, max_swaps);
  cache_fill_kernel<<<grid, kFillThreads, 0, s>>>(static_cast<const uint8_t*>(host_pool_dev),
                                                  host_n_slots, static_cast<uint8_t*>(pool),
                                                  n_slots, slot_bytes, swaps, n_swaps);
  return hipGetLastError();
}

hipError_t launch_cache_commit(int32_t* slot_of_expert, int E, const int32_t* swaps,
                               const int32_t* n_swaps, int max_swaps, hipStream_t s) {
  cache_commit_kernel<<<(max_swaps + 255) / 256, 256, 0, s>>>(slot_of_expert, E, swaps, n_swaps,
                                                               max_swaps);
  return hipGetLastError();
}

}  // namespace bitffn
