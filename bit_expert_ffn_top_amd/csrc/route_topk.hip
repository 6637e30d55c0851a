// Router top-k: one 64-wide wavefront per token.
//
// Each lane keeps NPL logits (expert e = lane + 64*j) as order-preserving
// 32-bit keys.  Each of the k rounds takes the wavefront maximum key with DPP
// row rotations plus four lane reads (no LDS traffic), then finds the
// smallest expert id holding that key with one ballot per register (ids grow
// with j first, then with the lane), and retires that entry.  The softmax
// over the k chosen logits is then taken across lanes 0..k-1.
#include "moe_internal.h"

namespace bitffn {
namespace {

__device__ __forceinline__ uint32_t orderable(float v) {
  if (v != v) v = -__builtin_huge_valf();  // NaN ranks as -inf
  if (v == 0.0f) v = 0.0f;                 // -0.0 ranks as +0.0
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float from_orderable(uint32_t u) {
  const uint32_t b = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __builtin_bit_cast(float, b);
}

template <int CTRL>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
  return o > v ? o : v;
}

// maximum over the wavefront, returned uniform
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v = max_dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v = max_dpp<0x124>(v);   // row_ror:4
  v = max_dpp<0x128>(v);   // row_ror:8
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int NPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T,
                                                   int E, int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wavefront
  const float* row = logits + static_cast<int64_t>(t) * E;

  // key 0 marks an empty entry: every real key is >= orderable(-inf) > 0
  uint32_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = e < E ? orderable(row[e]) : 0u;
  }

  float my_val = 0.0f;
  int my_idx = 0;
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int j = 1; j < NPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u32(best);
    int winner = 0;
#pragma unroll
    for (int j = NPL - 1; j >= 0; --j) {  // smallest id: lowest j, then lowest lane
      const uint64_t bal = __ballot(key[j] == best);
      if (bal) winner = 64 * j + __builtin_ctzll(bal);
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (lane + 64 * j == winner) key[j] = 0u;
    if (lane == r) {
      my_idx = winner;
      my_val = from_orderable(best);
    }
  }

  const float v0 = __shfl(my_val, 0, 64);
  float ex = 0.0f;
  if (lane < k) ex = expf(my_val == v0 ? 0.0f : my_val - v0);
  const float sum = wave_sum(ex);
  if (lane < k) {
    idx[static_cast<int64_t>(t) * k + lane] = my_idx;
    w[static_cast<int64_t>(t) * k + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx,
                             float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 block(256);
  const dim3 grid((T + 3) / 4);
  if (E <= 64)
    topk_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 128)
    topk_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 256)
    topk_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 512)
    topk_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  else
    topk_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace bitffn
