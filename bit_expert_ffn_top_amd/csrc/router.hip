// Router projection for a decode or verify step (T <= 4 tokens): one logit
// per routed expert from each token's hidden state, logits[t][e] =
// sum_j x[t][j] * W[e][j], with W in bfloat16, [E][d] row-major.
//
// One wavefront per expert row.  Lane l takes the 16-byte pieces of the row
// at elements 512c + 8l (c = 0..3 for d <= 2048) and the matching 8 values of
// every token (x, which the L2 serves to all workgroups after the first), all
// requested before any arithmetic; each piece's 8 weights multiply the 8
// values of each token.  A lane sums its products in element order, then the
// wavefront adds its 64 lane sums in a fixed butterfly, so every run gives
// the same bits.
// The row bytes are streamed once: nontemporal loads.  Bound: HBM (the
// weights, 2 bytes per element; x and the logits are small).
#include "moe_internal.h"

namespace bitffn {
namespace {

constexpr int RG_ROWS = 2;       // expert rows (wavefronts) per workgroup
constexpr int RG_CHUNK = 512;    // elements of a row covered by one pass of 64 lanes
constexpr int RG_PASSES = 4;     // passes for d <= 2048

typedef uint32_t ru4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

__global__ __launch_bounds__(RG_ROWS * 64) void router_gemv_kernel(
    const float* __restrict__ x, int T, int d, const uint16_t* __restrict__ w, int E,
    float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = static_cast<int>(blockIdx.x) * RG_ROWS + (static_cast<int>(threadIdx.x) >> 6);
  if (e >= E) return;   // uniform per wavefront
  const uint16_t* __restrict__ row = w + static_cast<int64_t>(e) * d;
  ru4 wv[RG_PASSES];
#pragma unroll
  for (int c = 0; c < RG_PASSES; ++c) {   // indices clamped into the row: every load in range
    const int j0 = min(RG_CHUNK * c + 8 * lane, d - 8);
    wv[c] = __builtin_nontemporal_load(reinterpret_cast<const ru4*>(row + j0));
  }
  // every token's matching x values, requested before any arithmetic too
  // (clamped indices; the surplus values are not used)
  float4 xv[MOE_MAX_DECODE_T][RG_PASSES][2];
#pragma unroll
  for (int t = 0; t < MOE_MAX_DECODE_T; ++t) {
    const float* __restrict__ xt = x + static_cast<int64_t>(t) * d;
#pragma unroll
    for (int c = 0; c < RG_PASSES; ++c) {
      const int j0 = min(RG_CHUNK * c + 8 * lane, d - 8);
      const bool here = t < T;   // uniform: only the T tokens' rows
      xv[t][c][0] = here ? *reinterpret_cast<const float4*>(xt + j0) : make_float4(0, 0, 0, 0);
      xv[t][c][1] = here ? *reinterpret_cast<const float4*>(xt + j0 + 4) : make_float4(0, 0, 0, 0);
    }
  }
  float acc[MOE_MAX_DECODE_T] = {};
#pragma unroll
  for (int c = 0; c < RG_PASSES; ++c) {
    if (RG_CHUNK * c + 8 * lane < d) {
      const float wf[8] = {bf16_lo(wv[c].x), bf16_hi(wv[c].x), bf16_lo(wv[c].y), bf16_hi(wv[c].y),
                           bf16_lo(wv[c].z), bf16_hi(wv[c].z), bf16_lo(wv[c].w), bf16_hi(wv[c].w)};
#pragma unroll
      for (int t = 0; t < MOE_MAX_DECODE_T; ++t) {
        const float4 x0 = xv[t][c][0], x1 = xv[t][c][1];
        float a = acc[t];
        a = fmaf(x0.x, wf[0], a);
        a = fmaf(x0.y, wf[1], a);
        a = fmaf(x0.z, wf[2], a);
        a = fmaf(x0.w, wf[3], a);
        a = fmaf(x1.x, wf[4], a);
        a = fmaf(x1.y, wf[5], a);
        a = fmaf(x1.z, wf[6], a);
        a = fmaf(x1.w, wf[7], a);
        acc[t] = a;
      }
    }
  }
#pragma unroll
  for (int t = 0; t < MOE_MAX_DECODE_T; ++t) {
    if (t < T) {
      float v = acc[t];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);   // same sum in every lane
      if (lane == 0) logits[static_cast<int64_t>(t) * E + e] = v;
    }
  }
}

}  // namespace

hipError_t launch_router_logits(const float* x, int T, int d, const uint16_t* w, int E,
                                float* logits, hipStream_t s) {
  const int grid = (E + RG_ROWS - 1) / RG_ROWS;
  router_gemv_kernel<<<grid, RG_ROWS * 64, 0, s>>>(x, T, d, w, E, logits);
  return hipGetLastError();
}

}  // namespace bitffn
