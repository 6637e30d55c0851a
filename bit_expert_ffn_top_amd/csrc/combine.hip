// Routing-weighted combine into the residual:
//   y[t] = x[t] + sum_i w[t,i] * rows[pair_pos[t,i]] + shared[t]
// One thread per 4 consecutive columns of one token; the k terms are added in
// i order with fused multiply-adds, the shared row last.  A missed pair
// (pair_pos < 0) contributes nothing.  The pair rows are read once and y is
// written once, both with nontemporal accesses (streamed past the caches).
#include "moe_internal.h"

namespace bitffn {
namespace {

typedef float nf4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_stream(const float* p) {
  const nf4 v = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}

template <bool XBF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ x, int T, int d,
                                                      int k, const float* __restrict__ rows,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ shared,
                                                      float* __restrict__ y) {
  const int d4 = d >> 2;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(T) * d4) return;
  const int t = static_cast<int>(gid / d4);
  const int c = static_cast<int>(gid - static_cast<int64_t>(t) * d4) * 4;
  float4 acc;
  if (XBF16) {
    const uint2 b = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) +
                                                    static_cast<int64_t>(t) * d + c);
    acc.x = bf16_bits_to_float(b.x & 0xFFFFu);
    acc.y = bf16_bits_to_float(b.x >> 16);
    acc.z = bf16_bits_to_float(b.y & 0xFFFFu);
    acc.w = bf16_bits_to_float(b.y >> 16);
  } else {
    acc = *reinterpret_cast<const float4*>(static_cast<const float*>(x) +
                                           static_cast<int64_t>(t) * d + c);
  }
  // the k terms in batches of KC: all pair positions and weights of a batch,
  // then all its row loads (a missed pair re-reads a row of the batch that is
  // present, so that every load is unconditional and in bounds, and is
  // skipped), then the fused multiply-adds in i order
  constexpr int KC = 10;
  for (int i0 = 0; i0 < k; i0 += KC) {
    int p[KC];
    float wi[KC];
    float4 r[KC];
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      const bool in = i0 + j < k;
      const int64_t q = static_cast<int64_t>(t) * k + min(i0 + j, k - 1);
      p[j] = in ? pair_pos[q] : -1;
      wi[j] = w[q];
    }
    int any = -1;
#pragma unroll
    for (int j = KC - 1; j >= 0; --j) any = p[j] >= 0 ? p[j] : any;
    if (any < 0) continue;   // the token's whole batch missed (uniform per wavefront)
#pragma unroll
    for (int j = 0; j < KC; ++j)
      r[j] = load_stream(rows + static_cast<int64_t>(p[j] >= 0 ? p[j] : any) * d + c);
#pragma unroll
    for (int j = 0; j < KC; ++j) {
      if (p[j] >= 0) {
        acc.x = fmaf(wi[j], r[j].x, acc.x);
        acc.y = fmaf(wi[j], r[j].y, acc.y);
        acc.z = fmaf(wi[j], r[j].z, acc.z);
        acc.w = fmaf(wi[j], r[j].w, acc.w);
      }
    }
  }
  if (shared) {
    const float4 r = *reinterpret_cast<const float4*>(shared + static_cast<int64_t>(t) * d + c);
    acc.x += r.x;
    acc.y += r.y;
    acc.z += r.z;
    acc.w += r.w;
  }
  const nf4 out = {acc.x, acc.y, acc.z, acc.w};
  __builtin_nontemporal_store(out, reinterpret_cast<nf4*>(y + static_cast<int64_t>(t) * d + c));
}

}  // namespace

hipError_t launch_combine(const void* x, int x_dtype, int T, int d, int k, const float* rows,
                          const int32_t* pair_pos, const float* w, const float* shared,
                          float* y, hipStream_t s) {
  const int64_t n = static_cast<int64_t>(T) * (d / 4);
  if (n == 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  if (x_dtype == MOE_DTYPE_BF16)
    combine_kernel<true><<<static_cast<unsigned>(blocks), 256, 0, s>>>(x, T, d, k, rows, pair_pos,
                                                                      w, shared, y);
  else
    combine_kernel<false><<<static_cast<unsigned>(blocks), 256, 0, s>>>(x, T, d, k, rows,
                                                                       pair_pos, w, shared, y);
  return hipGetLastError();
}

}  // namespace bitffn
