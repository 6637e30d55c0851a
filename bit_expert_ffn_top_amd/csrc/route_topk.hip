// Router top-k: one 64-wide wavefront per token.
//
// Each lane keeps NPL candidate keys (expert e = lane + 64*j).  A key packs
// the logit into an order-preserving 32-bit integer (high word) and the
// complement of the expert id (low word), so the unsigned 64-bit maximum is
// the largest logit with the smallest id.  k rounds of a wavefront max-reduce
// pick the experts in rank order; the winner's lane retires the key.  The
// softmax over the k chosen logits is then taken across lanes 0..k-1.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, 64);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, 64);
    const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
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

  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    key[j] = 0;
    if (e < E) {
      key[j] = (static_cast<uint64_t>(orderable(row[e])) << 32) | static_cast<uint32_t>(~e);
    }
  }

  float my_val = 0.0f;
  int my_idx = 0;
  for (int r = 0; r < k; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < NPL; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (key[j] == best) key[j] = 0;
    if (lane == r) {
      my_idx = static_cast<int>(~static_cast<uint32_t>(best));
      my_val = from_orderable(static_cast<uint32_t>(best >> 32));
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
