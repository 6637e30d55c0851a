// Router top-k: one workgroup per token, one wavefront per group of 64
// experts; the two-level rank selection and the softmax over the k chosen
// logits are the shared routing building blocks (also used by the fused
// decode layer, so both give identical bits).
#include "moe_internal.h"
#include "route_device.h"

namespace bitffn {
namespace {

constexpr int kMaxGroups = MOE_MAX_EXPERTS / 64;

__global__ __launch_bounds__(kMaxGroups * 64) void route_topk_kernel(
    const float* __restrict__ logits, int E, int k, int32_t* __restrict__ idx,
    float* __restrict__ w) {
  __shared__ uint64_t grp[kMaxGroups * 64];
  __shared__ uint64_t cand[kMaxGroups * MOE_MAX_TOPK];
  __shared__ uint64_t top[MOE_MAX_TOPK];
  const int64_t t = blockIdx.x;
  block_topk<1>(logits + t * E, 1, E, k, TopkLds{grp, cand, top});
  if (threadIdx.x < 64) {
    int id;
    float wt;
    topk_softmax_lane(top, k, threadIdx.x, id, wt);
    if (static_cast<int>(threadIdx.x) < k) {
      idx[t * k + threadIdx.x] = id;
      w[t * k + threadIdx.x] = wt;
    }
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* idx,
                             float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int groups = (E + 63) / 64;   // <= kMaxGroups: every group has its wavefront
  route_topk_kernel<<<T, groups * 64, 0, s>>>(logits, E, k, idx, w);
  return hipGetLastError();
}

}  // namespace bitffn
