// Device building blocks of routing, shared by the standalone route/lookup
// kernels and the fused decode layer, so both produce identical bits.
//
// Order of experts (value desc, index asc), with -0.0 ranked as +0.0 and NaN
// as -inf, is carried by one 64-bit key: the order-preserving image of the
// logit in the high word and the complemented expert id in the low word.
// Distinct experts have distinct keys, so every rank is a count of larger
// keys, and one unsigned compare decides each pair.
//
// Top-k, two levels, all in LDS:
//   1. groups of 64 experts: each key's rank within its group (64 compares
//      against the group's keys); keys ranked below k survive, at position
//      group*k + rank;
//   2. each survivor's rank among the G*k survivors of its token; a survivor
//      with rank r < k is the token's r-th choice.
// The k-th largest key of a token is among the k largest of its own group,
// so nothing that belongs to the top k is dropped in step 1.
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

// LDS scratch of block_topk for T tokens of E experts, top k:
//   grp  [nwaves * 64]   per-wavefront group keys
//   cand [T * G * k]     survivors of step 1, G = ceil(E / 64)
//   top  [T * k]         result keys in rank order
struct TopkLds {
  uint64_t* grp;
  uint64_t* cand;
  uint64_t* top;
};

// Top-k keys of T tokens, called by every thread of the workgroup (blockDim.x
// a multiple of 64).  Wavefront w handles groups w, w + nwaves, ...; MAXIT
// bounds the groups per wavefront: T * G <= MAXIT * nwaves.
//
// topk_load requests the logits of the wavefront's groups (clamped indices:
// every load is in range and unconditional); topk_select ranks them.  `hook`
// runs in every thread just before the first barrier (callers use it to
// store data that must be visible after the selection).  Ends with a
// barrier; the result is in s.top.
template <int MAXIT>
__device__ __forceinline__ void topk_load(const float* __restrict__ logits, int T, int E,
                                          float (&lg)[MAXIT]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int G = (E + 63) >> 6;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int q = min(wave + it * nwaves, T * G - 1);
    const int t = q / G, e = (q - t * G) * 64 + lane;
    lg[it] = logits[static_cast<int64_t>(t) * E + min(e, E - 1)];
  }
}

template <int MAXIT, typename Hook>
__device__ __forceinline__ void topk_select(const float (&lg)[MAXIT], int T, int E, int k,
                                            const TopkLds& s, Hook&& hook) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwaves = blockDim.x >> 6;
  const int G = (E + 63) >> 6;
  uint64_t* grp = s.grp + wave * 64;
#pragma unroll
  for (int it = 0; it < MAXIT; ++it) {
    const int q = wave + it * nwaves;
    if (q < T * G) {   // uniform
      const int t = q / G, g = q - t * G, e = g * 64 + lane;
      const uint64_t key = route_key(lg[it], e, e < E);
      grp[lane] = key;
      __builtin_amdgcn_wave_barrier();
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < 64; ++j) rank += grp[j] > key ? 1 : 0;
      if (rank < k) s.cand[(t * G + g) * k + rank] = key;
      __builtin_amdgcn_wave_barrier();
    }
  }
  hook();
  __syncthreads();

  const int C = G * k;
  for (int c = tid; c < T * C; c += blockDim.x) {
    const uint64_t* cand = s.cand + (c / C) * C;
    const uint64_t key = s.cand[c];
    int rank = 0;
    for (int j = 0; j < C; ++j) rank += cand[j] > key ? 1 : 0;
    if (rank < k) s.top[(c / C) * k + rank] = key;
  }
  __syncthreads();
}

template <int MAXIT>
__device__ __forceinline__ void block_topk(const float* __restrict__ logits, int T, int E, int k,
                                           const TopkLds& s) {
  float lg[MAXIT];
  topk_load<MAXIT>(logits, T, E, lg);
  topk_select<MAXIT>(lg, T, E, k, s, [] {});
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
