// Router top-k, one wavefront per token: lane l holds the keys of experts
// 64j + l (the 64-bit keys of the shared routing building blocks: value desc,
// index asc, -0 as +0, NaN as -inf; all distinct), and the fused decode
// layer's selection (a bound from the lane maxima, the candidates at or above
// it ranked among themselves) gives choice r = the key of rank r.  The softmax
// over the k chosen logits is the shared one, so both give identical bits.
#include "moe_internal.h"
#include "route_device.h"

namespace bitffn {
namespace {

constexpr int kTokensPerBlock = 4;   // one wavefront each

template <int M>   // keys per lane: E <= 64 * M
__global__ __launch_bounds__(64 * kTokensPerBlock) void route_topk_kernel(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ idx,
    float* __restrict__ w) {
  __shared__ uint64_t top[kTokensPerBlock][MOE_MAX_TOPK];
  __shared__ uint64_t scratch[kTokensPerBlock][128];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + wave;
  if (t >= T) return;   // uniform per wavefront; no barrier follows
  const float* lg = logits + t * E;
  uint64_t key[M];
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const int e = 64 * j + lane;
    key[j] = route_key(lg[min(e, E - 1)], e, e < E);
  }
  wave_topk_keys<M>(key, k, top[wave], scratch[wave]);
  int id;
  float wt;
  topk_softmax_lane(top[wave], k, lane, id, wt);
  if (lane < k) {
    idx[t * k + lane] = id;
    w[t * k + lane] = wt;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx,
                             float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int blocks = (T + kTokensPerBlock - 1) / kTokensPerBlock;
  const int threads = 64 * kTokensPerBlock;
  const int m = (E + 63) / 64;   // E <= MOE_MAX_EXPERTS = 1024: m <= 16
  if (m <= 2)
    route_topk_kernel<2><<<blocks, threads, 0, s>>>(logits, T, E, k, idx, w);
  else if (m <= 4)
    route_topk_kernel<4><<<blocks, threads, 0, s>>>(logits, T, E, k, idx, w);
  else if (m <= 8)
    route_topk_kernel<8><<<blocks, threads, 0, s>>>(logits, T, E, k, idx, w);
  else
    route_topk_kernel<16><<<blocks, threads, 0, s>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace bitffn
