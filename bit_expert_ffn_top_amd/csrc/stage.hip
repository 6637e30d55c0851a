// Staging of a whole layer for a prefill chunk: every expert's packed slot is
// copied into a staging pool in expert order (slot e = expert e, slot E = the
// shared expert), the resident ones from the GPU cache and the others from
// the host tier.  Copies go through hipMemcpyAsync, so the DMA engines move
// the bytes while the compute units run the previous layer's GEMMs; runs of
// experts whose source slots are consecutive are merged into one copy.
#include "moe_internal.h"

namespace bitffn {

hipError_t launch_stage_layer(const moe_layer& C, const int32_t* slot_of_expert,
                              const void* host_pool, const int32_t* host_slot_of_expert,
                              void* staging, hipStream_t s) {
  const int E = C.n_experts;
  const int64_t sb = C.slot_bytes;
  const uint8_t* cache = static_cast<const uint8_t*>(C.pool);
  const uint8_t* host = static_cast<const uint8_t*>(host_pool);
  uint8_t* dst = static_cast<uint8_t*>(staging);
  // source of expert e (E: the shared expert)
  auto source = [&](int e) -> const uint8_t* {
    if (e == E) return cache + static_cast<int64_t>(C.shared_slot) * sb;
    const int cs = slot_of_expert[e];
    if (cs >= 0) return cache + static_cast<int64_t>(cs) * sb;
    return host + static_cast<int64_t>(host_slot_of_expert[e]) * sb;
  };
  const int last = C.shared_slot >= 0 ? E : E - 1;
  int e0 = 0;
  while (e0 <= last) {
    const uint8_t* src0 = source(e0);
    int e1 = e0 + 1;
    while (e1 <= last && source(e1) == src0 + static_cast<int64_t>(e1 - e0) * sb) ++e1;
    const hipError_t err = hipMemcpyAsync(dst + static_cast<int64_t>(e0) * sb, src0,
                                          static_cast<size_t>((e1 - e0) * sb), hipMemcpyDefault, s);
    if (err != hipSuccess) return err;
    e0 = e1;
  }
  return hipSuccess;
}

}  // namespace bitffn
