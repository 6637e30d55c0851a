// Device building blocks of routing, shared by the standalone route/lookup
// kernels and the fused decode layer, so both produce identical bits.
//
// Order of experts (value desc, index asc), with -0.0 ranked as +0.0 and NaN
// as -inf, is carried by one 64-bit key: the order-preserving image of the
// logit in the high word and the complemented expert id in the low word.
// Distinct experts have distinct keys, so every rank is a count of larger
// keys, and one unsigned compare decides each pair.
//
// Top-k of one token in one wavefront (wave_topk_keys): a lower bound from the
// lane maxima, the candidates at or above it gathered and ranked among
// themselves; every rank is a count of larger keys, so any correct selection
// gives the same keys in the same order.
#pragma once

#include "moe_common.h"

namespace bitffn {

__device__ __forceinline__ uint32_t orderable_bits(float v) {
  if (v != v) v = -__builtin_huge_valf();  // NaN ranks as -inf
  if (v == 0.0f) v = 0.0f;                 // -0.0 ranks as +0.0
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float from_orderable_bits(uint32_t u) {
  const uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __builtin_bit_cast(float, b);
}

// Key of expert e with logit v; an absent expert (e >= E) gets a key below
// every real one (high word 0) that is still unique.
__device__ __forceinline__ uint64_t route_key(float v, int e, bool present) {
  const uint64_t lo = static_cast<uint32_t>(~static_cast<uint32_t>(e));
  return present ? ((static_cast<uint64_t>(orderable_bits(v)) << 32) | lo) : lo;
}

__device__ __forceinline__ int key_expert(uint64_t key) {
  return static_cast<int>(~static_cast<uint32_t>(key));
}

__device__ __forceinline__ float key_value(uint64_t key) {
  return from_orderable_bits(static_cast<uint32_t>(key >> 32));
}

__device__ __forceinline__ float route_wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// A lower bound of the k-th largest of one 32-bit value per lane (k <= 64):
// the largest tau whose low LOW bits are zero with at least k values >= tau,
// found bit by bit with ballot counts (the k-th largest itself for LOW = 0).
template <int LOW = 0>
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t v, int k) {
  uint32_t tau = 0;
#pragma unroll
  for (int b = 31; b >= LOW; --b) {
    const uint32_t cand = tau | (1u << b);
    if (__popcll(__ballot(v >= cand)) >= k) tau = cand;
  }
  return tau;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// k rounds of the wavefront's largest remaining key (lane-local maximum, then
// a butterfly of 64-bit maxima); the winner is removed.  top[r] = key of rank r.
template <int NJ>
__device__ __forceinline__ void wave_topk_rounds(uint64_t (&key)[NJ], int k, uint64_t* top) {
  const int lane = threadIdx.x & 63;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < NJ; ++j) best = key[j] > best ? key[j] : best;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const uint64_t o = __shfl_xor(best, off, 64);
      best = o > best ? o : best;
    }
    if (lane == 0) top[r] = best;
#pragma unroll
    for (int j = 0; j < NJ; ++j) key[j] = key[j] == best ? 0ull : key[j];   // keys are never 0
  }
}

// Top-k keys of one token in one whole wavefront: lane l holds the keys of
// experts 64j + l (j < NJ; key = orderable value << 32 | ~id, 0 for experts
// >= E, below every real key).  A bound first: tau0, the k-th largest of the
// 64 lane maxima (by value) with its low 16 bits cleared, has at least k keys
// whose value is >= tau0, and the k-th largest key is at least the k-th
// largest lane maximum, so the top k are among them.  Those candidates
// (usually a little over k) are gathered into scratch in (j, lane) order and
// ranked among themselves by (value desc, id asc); the first k, in rank
// order, go to top[0..k).  Up to 16 candidates, every lane reads all 16
// slots at once and counts the larger keys (no serial chain of lane reads);
// up to 64, one lane read per candidate; past 64 (many equal values), k
// rounds of the largest remaining key.  scratch: 128 uint64 of LDS for this
// wavefront (slots 64 + lane take the writes of lanes without a candidate,
// so the gather needs no branch).  Same keys, same order as ranking every key.
template <int NJ>
__device__ __forceinline__ void wave_topk_keys(uint64_t (&key)[NJ], int k, uint64_t* top,
                                               uint64_t* scratch) {
  constexpr int kDirect = 16;
  const int lane = threadIdx.x & 63;
  uint32_t m = static_cast<uint32_t>(key[0] >> 32);   // lane maximum of the values
#pragma unroll
  for (int j = 1; j < NJ; ++j) m = max(m, static_cast<uint32_t>(key[j] >> 32));
  const uint32_t tau0 = wave_kth_largest<16>(m, k);
  const uint64_t below = (1ull << lane) - 1ull;
  // gather and count in one pass; candidates past the 64th are not stored
  int n_c = 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const bool c = static_cast<uint32_t>(key[j] >> 32) >= tau0;
    const uint64_t sel = __ballot(c);
    const int at = n_c + __popcll(sel & below);
    scratch[c && at < 64 ? at : 64 + lane] = key[j];
    n_c += __popcll(sel);
  }
  __builtin_amdgcn_wave_barrier();
  if (n_c <= kDirect) {
    const uint64_t mine = lane < n_c ? scratch[lane] : 0ull;
    uint64_t other[kDirect];
#pragma unroll
    for (int q = 0; q < kDirect; ++q) other[q] = scratch[q];   // same address in every lane
    int rank = 0;
#pragma unroll
    for (int q = 0; q < kDirect; ++q) rank += q < n_c && other[q] > mine ? 1 : 0;
    __builtin_amdgcn_wave_barrier();
    if (lane < n_c && rank < k) top[rank] = mine;
  } else if (n_c <= 64) {
    const uint64_t mine = lane < n_c ? scratch[lane] : 0ull;
    int rank = 0;
    for (int q = 0; q < n_c; ++q) rank += readlane_u64(mine, q) > mine ? 1 : 0;
    __builtin_amdgcn_wave_barrier();
    if (lane < n_c && rank < k) top[rank] = mine;
  } else {
    wave_topk_rounds<NJ>(key, k, top);
  }
  __builtin_amdgcn_wave_barrier();
}

// Routing weights of one token from its top keys (called by one whole
// wavefront; lane r < k gets choice r): w_r = exp(l_r - l_0) / sum_j exp(l_j - l_0),
// summed in a fixed xor tree.
__device__ __forceinline__ void topk_softmax_lane(const uint64_t* top, int k, int lane,
                                                  int& id, float& w) {
  const float v0 = key_value(top[0]);
  float ex = 0.0f;
  id = 0;
  if (lane < k) {
    const uint64_t key = top[lane];
    const float v = key_value(key);
    id = key_expert(key);
    ex = expf(v == v0 ? 0.0f : v - v0);
  }
  const float sum = route_wave_sum(ex);
  w = ex / sum;
}

// Miss lists of n <= 64 pairs, one whole wavefront, lane p = pair p with
// expert e and slot s: miss_pair in (expert, pair) order, miss_expert the
// ascending distinct missed experts, n_miss = {distinct, pairs}.  Pairs are
// compared through lane reads, so there is no LDS traffic.
__device__ __forceinline__ void wave_miss_lists(int p, int n, int e, int s,
                                                int32_t* __restrict__ miss_expert,
                                                int32_t* __restrict__ miss_pair,
                                                int32_t* __restrict__ n_miss) {
  const bool miss = p < n && s < 0;
  const int key = miss ? e : 0x7FFFFFFF;   // only missed pairs take part
  int pos = 0;          // missed pairs before this one in (expert, pair) order
  int dpos = 0;         // distinct missed experts with a smaller id
  bool first = miss;    // first missed pair naming this expert
  for (int q = 0; q < n; ++q) {
    const int kq = __builtin_amdgcn_readlane(key, q);
    if (kq == 0x7FFFFFFF) continue;
    pos += (kq < key || (kq == key && q < p)) ? 1 : 0;
    if (kq == key && q < p) first = false;
  }
  const uint64_t firsts = __ballot(first);
  for (int q = 0; q < n; ++q) {
    if (!((firsts >> q) & 1ull)) continue;
    const int kq = __builtin_amdgcn_readlane(key, q);
    dpos += kq < key ? 1 : 0;
  }
  const uint64_t misses = __ballot(miss);   // taken by the whole wavefront
  if (miss && miss_pair) miss_pair[pos] = p;
  if (first) miss_expert[dpos] = e;
  if (p == 0) {
    n_miss[0] = __popcll(firsts);
    n_miss[1] = __popcll(misses);
  }
}

}  // namespace bitffn
