// Decode / verify through a stack of MoE layers: per layer one routed FFN
// kernel and one combine kernel (the two launches of moe_decode_layer), where
// the combine also forms the next layer's input x' = y + addend, so layer l+1
// starts from layer l's finished output.  Every reduction of both kernels has
// a fixed order, so the step is bitwise reproducible and a token verified
// with drafts gets the bits it gets alone.
//
// Workspace: the decode layer's partial products (reused by every layer), two
// input buffers the layers alternate between, and stand-ins for the outputs
// the caller did not ask for (routing outputs, intermediate y).
#include "moe_internal.h"

namespace bitffn {

namespace {

struct StackWs {
  uint8_t* part;
  float* xbuf[2];
  int32_t* idx;
  float* w;
  int32_t* slot;
  int32_t* miss_expert;
  int32_t* n_miss;
};

int64_t a256(int64_t n) { return (n + 255) & ~int64_t(255); }

StackWs stack_ws(uintptr_t base, const StackDims& D, size_t* total) {
  StackWs w{};
  uintptr_t p = base;
  const int64_t xs = a256(static_cast<int64_t>(D.T) * D.d * 4);
  const int64_t pairs = a256(static_cast<int64_t>(D.T) * D.k * 4);
  w.part = reinterpret_cast<uint8_t*>(p);
  p += a256(static_cast<int64_t>(decode_workspace_bytes(D.d, D.f, D.T, D.k)));
  w.xbuf[0] = reinterpret_cast<float*>(p);
  p += xs;
  w.xbuf[1] = reinterpret_cast<float*>(p);
  p += xs;
  w.idx = reinterpret_cast<int32_t*>(p);
  p += pairs;
  w.w = reinterpret_cast<float*>(p);
  p += pairs;
  w.slot = reinterpret_cast<int32_t*>(p);
  p += pairs;
  w.miss_expert = reinterpret_cast<int32_t*>(p);
  p += pairs;
  w.n_miss = reinterpret_cast<int32_t*>(p);
  p += 256;
  if (total) *total = static_cast<size_t>(p - base);
  return w;
}

}  // namespace

size_t decode_stack_workspace_bytes(int d, int f, int T, int k) {
  size_t total = 0;
  stack_ws(0, StackDims{d, f, 0, k, T}, &total);
  return total;
}

hipError_t launch_decode_stack(const StackDims& D, int n_layers, const moe_stack_layer* layers,
                               const float* x, void* ws, hipStream_t s) {
  const StackWs w = stack_ws(reinterpret_cast<uintptr_t>(ws), D, nullptr);
  const float* xl = x;
  for (int l = 0; l < n_layers; ++l) {
    const moe_stack_layer& S = layers[l];
    moe_layer L{};
    L.d_model = D.d;
    L.d_ff = D.f;
    L.n_experts = D.E;
    L.top_k = D.k;
    L.fmt = S.fmt;
    L.n_slots = S.n_slots;
    L.shared_slot = S.shared_slot;
    L.reserved = 0;
    L.slot_bytes = S.slot_bytes;
    L.pool = S.pool;
    const bool last = l + 1 == n_layers;
    float* xnext = last ? nullptr : w.xbuf[l & 1];
    const float* addend = last ? nullptr : layers[l + 1].addend;
    const bool routing = S.idx != nullptr;
    const bool misses = S.miss_expert != nullptr;
    const hipError_t e = launch_decode_layer(
        L, xl, D.T, S.logits, S.slot_of_expert, routing ? S.idx : w.idx, routing ? S.w : w.w,
        routing ? S.slot : w.slot, misses ? S.miss_expert : w.miss_expert,
        misses ? S.miss_pair : nullptr, misses ? S.n_miss : w.n_miss, S.y, w.part, s, xnext,
        addend);
    if (e != hipSuccess) return e;
    xl = xnext;
  }
  return hipSuccess;
}

}  // namespace bitffn
