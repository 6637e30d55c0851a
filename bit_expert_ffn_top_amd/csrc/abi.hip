// C ABI entry points: host-side argument checks, workspace sizing, dispatch.
// Nothing here allocates; every check runs before the first HIP call.
#include <stdint.h>

#include "bitffn_moe.h"
#include <atomic>

#include "moe_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = static_cast<int>(e);
  return MOE_EHIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

bool valid_dims(int fmt, int d, int f) {
  (void)fmt;
  if (d < 64 || d > 2048 || d % 64 != 0) return false;
  if (f < 32 || f > 4096 || f % 32 != 0) return false;
  return true;
}

// Scratch of moe_decode_layer_noalloc: a file-scope device array, one copy
// per GPU, kept until the process ends.  Host code never passes the array's
// name to a kernel (that is a host-side stand-in); it asks the runtime for
// each device's address once, with that device current, and uses that.
constexpr size_t kNoAllocScratchBytes = size_t{16} << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices] = {};

// This device's address of `scratch` (looked up on the first call per
// device); nullptr with *err set when the lookup fails.
void* scratch_address(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kScratchDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

bool valid_fmt(int fmt) {
  return fmt == MOE_FMT_Q2S || fmt == MOE_FMT_Q2SM || fmt == MOE_FMT_Q3G;
}

int check_layer(const moe_layer* L) {
  if (!L) return MOE_EINVAL;
  if (!valid_fmt(L->fmt)) return MOE_EFORMAT;
  if (!valid_dims(L->fmt, L->d_model, L->d_ff)) return MOE_EINVAL;
  if (L->n_experts < 1 || L->n_experts > MOE_MAX_EXPERTS) return MOE_EINVAL;
  if (L->top_k < 1 || L->top_k > MOE_MAX_TOPK || L->top_k > L->n_experts) return MOE_EINVAL;
  if (L->n_slots < 1) return MOE_EINVAL;
  if (L->shared_slot < -1 || L->shared_slot >= L->n_slots) return MOE_EINVAL;
  if (L->reserved != 0) return MOE_EINVAL;
  if (L->slot_bytes != bitffn::slot_layout(L->fmt, L->d_model, L->d_ff).total) return MOE_EFORMAT;
  if (!L->pool) return MOE_EINVAL;
  if (!aligned256(L->pool)) return MOE_EALIGN;
  return MOE_OK;
}

// Device-side address of memory this device can read: pinned host memory
// (hipHostMalloc) or device memory.  False for anything else (pageable host
// memory), leaving no HIP error behind.
bool device_address(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (!attr.devicePointer || (attr.type != hipMemoryTypeHost && attr.type != hipMemoryTypeDevice))
    return false;
  *out = attr.devicePointer;
  return true;
}

// The checks of moe_decode_layer's arguments other than the workspace.
int check_decode_layer(const moe_layer* L, const float* x, int T, const float* logits,
                       const int32_t* slot_of_expert, const int32_t* idx, const float* w,
                       const int32_t* slot, const int32_t* miss_expert, const int32_t* miss_pair,
                       const int32_t* n_miss, const float* y) {
  const int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 1 || T > MOE_MAX_DECODE_T || T * L->top_k > MOE_MAX_DECODE_PAIRS) return MOE_EINVAL;
  if (!x || !logits || !slot_of_expert || !idx || !w || !slot || !miss_expert || !n_miss || !y)
    return MOE_EINVAL;
  if (static_cast<const void*>(x) == static_cast<const void*>(y)) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(logits) || !aligned16(slot_of_expert) || !aligned16(idx) ||
      !aligned16(w) || !aligned16(slot) || !aligned16(miss_expert) || !aligned16(n_miss) ||
      (miss_pair && !aligned16(miss_pair)) || !aligned16(y))
    return MOE_EALIGN;
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EALIGN: return "misaligned device pointer";
    case MOE_EFORMAT: return "unknown block format or slot size mismatch";
    case MOE_ENOSPC: return "workspace too small";
    case MOE_EHIP: return "HIP call failed";
    default: return "unknown status";
  }
}

int moe_last_hip_error(void) { return g_last_hip_error; }

int64_t moe_slot_bytes(int fmt, int d_model, int d_ff) {
  if (!valid_fmt(fmt)) return MOE_EFORMAT;
  if (!valid_dims(fmt, d_model, d_ff)) return MOE_EINVAL;
  return bitffn::slot_layout(fmt, d_model, d_ff).total;
}

int moe_router_logits(const float* x, int T, int d_model, const uint16_t* w, int n_experts,
                      float* logits, hipStream_t stream) {
  if (T < 1 || T > MOE_MAX_DECODE_T) return MOE_EINVAL;
  if (d_model < 64 || d_model > 2048 || d_model % 64 != 0) return MOE_EINVAL;
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return MOE_EINVAL;
  if (!x || !w || !logits) return MOE_EINVAL;
  if (static_cast<const void*>(logits) == static_cast<const void*>(x) ||
      static_cast<const void*>(logits) == static_cast<const void*>(w))
    return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w) || !aligned16(logits)) return MOE_EALIGN;
  return hip_status(bitffn::launch_router_logits(x, T, d_model, w, n_experts, logits, stream));
}

int moe_route_topk(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                   hipStream_t stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK || k > E) return MOE_EINVAL;
  if (T < 0 || T >= (1 << 24)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!logits || !idx || !w) return MOE_EINVAL;
  if (!aligned16(logits) || !aligned16(idx) || !aligned16(w)) return MOE_EALIGN;
  return hip_status(bitffn::launch_route_topk(logits, T, E, k, idx, w, stream));
}

size_t moe_lookup_workspace_bytes(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1 || E > MOE_MAX_EXPERTS) return 0;
  if (static_cast<int64_t>(T) * k <= bitffn::kSmallLookupPairs) return 0;
  return bitffn::group_workspace_bytes(T, E);
}

int moe_cache_lookup(const int32_t* idx, int T, int k, const int32_t* slot_of_expert, int E,
                     int32_t* slot, int32_t* miss_expert, int32_t* miss_pair, int32_t* n_miss,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || k < 1 || k > MOE_MAX_TOPK) return MOE_EINVAL;
  if (T < 0 || T > 65536) return MOE_EINVAL;
  if (!idx || !slot_of_expert || !slot || !miss_expert || !n_miss) return MOE_EINVAL;
  if (!aligned16(idx) || !aligned16(slot_of_expert) || !aligned16(slot) ||
      !aligned16(miss_expert) || !aligned16(n_miss) || (miss_pair && !aligned16(miss_pair)))
    return MOE_EALIGN;
  const int64_t n = static_cast<int64_t>(T) * k;
  if (n <= bitffn::kSmallLookupPairs)
    return hip_status(bitffn::launch_lookup_small(idx, T, k, slot_of_expert, E, slot,
                                                  miss_expert, miss_pair, n_miss, stream));
  if (!ws) return MOE_EINVAL;
  if (!aligned256(ws)) return MOE_EALIGN;
  if (ws_bytes < bitffn::group_workspace_bytes(T, E)) return MOE_ENOSPC;
  // slot for every pair, then the grouping of the missed pairs
  hipError_t e = bitffn::launch_lookup_slots(idx, T, k, slot_of_expert, slot, stream);
  if (e != hipSuccess) return hip_status(e);
  const bitffn::GroupWorkspace gws = bitffn::group_workspace(ws, T, E);
  return hip_status(bitffn::launch_group_pairs(idx, slot, nullptr, T, k, E, false, 0, gws, nullptr,
                                               miss_pair, nullptr, miss_expert, n_miss, nullptr,
                                               0, nullptr, nullptr, stream));
}

size_t moe_decode_workspace_bytes(const moe_layer* L, int T) {
  if (check_layer(L) != MOE_OK || T < 1 || T > MOE_MAX_DECODE_T) return 0;
  return bitffn::decode_workspace_bytes(L->d_model, L->d_ff, T, L->top_k);
}

int moe_expert_ffn_decode(const moe_layer* L, const float* x, int T, const int32_t* idx,
                          const int32_t* slot, const float* w, float* y, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  const int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 1 || T > MOE_MAX_DECODE_T || T * L->top_k > MOE_MAX_DECODE_PAIRS) return MOE_EINVAL;
  if (!x || !idx || !slot || !w || !y || !ws) return MOE_EINVAL;
  if (static_cast<const void*>(x) == static_cast<const void*>(y)) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(idx) || !aligned16(slot) || !aligned16(w) || !aligned16(y))
    return MOE_EALIGN;
  if (!aligned256(ws)) return MOE_EALIGN;
  if (ws_bytes < bitffn::decode_workspace_bytes(L->d_model, L->d_ff, T, L->top_k))
    return MOE_ENOSPC;
  return hip_status(bitffn::launch_decode(*L, x, T, idx, slot, w, y, ws, stream));
}

int moe_decode_layer(const moe_layer* L, const float* x, int T, const float* logits,
                     const int32_t* slot_of_expert, int32_t* idx, float* w, int32_t* slot,
                     int32_t* miss_expert, int32_t* miss_pair, int32_t* n_miss, float* y,
                     void* ws, size_t ws_bytes, hipStream_t stream) {
  const int st = check_decode_layer(L, x, T, logits, slot_of_expert, idx, w, slot, miss_expert,
                                    miss_pair, n_miss, y);
  if (st != MOE_OK) return st;
  if (!ws) return MOE_EINVAL;
  if (!aligned256(ws)) return MOE_EALIGN;
  if (ws_bytes < bitffn::decode_workspace_bytes(L->d_model, L->d_ff, T, L->top_k))
    return MOE_ENOSPC;
  return hip_status(bitffn::launch_decode_layer(*L, x, T, logits, slot_of_expert, idx, w, slot,
                                                miss_expert, miss_pair, n_miss, y, ws, stream));
}

int moe_decode_layer_noalloc(const moe_layer* L, const float* x, int T, const float* logits,
                             const int32_t* slot_of_expert, int32_t* idx, float* w,
                             int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                             int32_t* n_miss, float* y, hipStream_t stream) {
  // every argument is checked before the first HIP call (the address lookup)
  const int st = check_decode_layer(L, x, T, logits, slot_of_expert, idx, w, slot, miss_expert,
                                    miss_pair, n_miss, y);
  if (st != MOE_OK) return st;
  if (bitffn::decode_workspace_bytes(L->d_model, L->d_ff, T, L->top_k) > kNoAllocScratchBytes)
    return MOE_ENOSPC;
  hipError_t e = hipSuccess;
  void* ws = scratch_address(&e);
  if (!ws) return hip_status(e);
  return moe_decode_layer(L, x, T, logits, slot_of_expert, idx, w, slot, miss_expert, miss_pair,
                          n_miss, y, ws, kNoAllocScratchBytes, stream);
}

int moe_decode_layer_tiers(const moe_layer* L, const moe_layer* H,
                           const int32_t* host_slot_of_expert, int max_rank, const float* x,
                           int T, const float* logits, const int32_t* slot_of_expert,
                           int32_t* idx, float* w, int32_t* slot, int32_t* miss_expert,
                           int32_t* miss_pair, int32_t* n_miss, float* y, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  int st = check_decode_layer(L, x, T, logits, slot_of_expert, idx, w, slot, miss_expert,
                              miss_pair, n_miss, y);
  if (st != MOE_OK) return st;
  st = check_layer(H);
  if (st != MOE_OK) return st;
  // the host tier holds slots of the same experts in the same format
  if (H->fmt != L->fmt || H->d_model != L->d_model || H->d_ff != L->d_ff ||
      H->n_experts != L->n_experts || H->top_k != L->top_k || H->shared_slot != -1)
    return MOE_EINVAL;
  if (max_rank < 0 || max_rank > L->top_k) return MOE_EINVAL;
  if (!host_slot_of_expert || !ws) return MOE_EINVAL;
  if (!aligned16(host_slot_of_expert) || !aligned256(ws)) return MOE_EALIGN;
  if (ws_bytes < bitffn::decode_workspace_bytes(L->d_model, L->d_ff, T, L->top_k))
    return MOE_ENOSPC;
  const void* host_dev = nullptr;
  if (!device_address(H->pool, &host_dev)) return MOE_EINVAL;
  return hip_status(bitffn::launch_decode_layer_tiers(*L, *H, host_dev, host_slot_of_expert,
                                                      max_rank, x, T, logits, slot_of_expert,
                                                      idx, w, slot, miss_expert, miss_pair,
                                                      n_miss, y, ws, stream));
}

size_t moe_decode_stack_workspace_bytes(int d_model, int d_ff, int n_experts, int top_k, int T) {
  if (!valid_dims(MOE_FMT_Q2SM, d_model, d_ff)) return 0;
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS || top_k < 1 || top_k > MOE_MAX_TOPK ||
      top_k > n_experts)
    return 0;
  if (T < 1 || T > MOE_MAX_DECODE_T || T * top_k > MOE_MAX_DECODE_PAIRS) return 0;
  return bitffn::decode_stack_workspace_bytes(d_model, d_ff, T, top_k);
}

int moe_decode_stack(int d_model, int d_ff, int n_experts, int top_k, int T, int n_layers,
                     const moe_stack_layer* layers, const float* x, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (!valid_dims(MOE_FMT_Q2SM, d_model, d_ff)) return MOE_EINVAL;
  if (n_experts < 1 || n_experts > MOE_MAX_EXPERTS || top_k < 1 || top_k > MOE_MAX_TOPK ||
      top_k > n_experts)
    return MOE_EINVAL;
  if (T < 1 || T > MOE_MAX_DECODE_T || T * top_k > MOE_MAX_DECODE_PAIRS) return MOE_EINVAL;
  if (n_layers < 1) return MOE_EINVAL;
  if (!layers || !x || !ws) return MOE_EINVAL;
  if (!aligned16(x) || !aligned256(ws)) return MOE_EALIGN;
  for (int l = 0; l < n_layers; ++l) {
    const moe_stack_layer& S = layers[l];
    if (!valid_fmt(S.fmt)) return MOE_EFORMAT;
    if (S.slot_bytes != bitffn::slot_layout(S.fmt, d_model, d_ff).total) return MOE_EFORMAT;
    if (S.n_slots < 1 || S.shared_slot < -1 || S.shared_slot >= S.n_slots || S.reserved != 0)
      return MOE_EINVAL;
    if (!S.pool || !S.slot_of_expert || !S.logits) return MOE_EINVAL;
    if (l + 1 == n_layers && !S.y) return MOE_EINVAL;
    const int routing = (S.idx ? 1 : 0) + (S.w ? 1 : 0) + (S.slot ? 1 : 0);
    if (routing != 0 && routing != 3) return MOE_EINVAL;
    if ((S.miss_expert != nullptr) != (S.n_miss != nullptr)) return MOE_EINVAL;
    if (S.miss_pair && !S.miss_expert) return MOE_EINVAL;
    if (!aligned256(S.pool)) return MOE_EALIGN;
    const void* ptrs[] = {S.slot_of_expert, S.logits, S.addend, S.y, S.idx, S.w, S.slot,
                          S.miss_expert, S.miss_pair, S.n_miss};
    for (const void* q : ptrs)
      if (q && !aligned16(q)) return MOE_EALIGN;
    if (S.y && static_cast<const void*>(S.y) == static_cast<const void*>(x)) return MOE_EINVAL;
  }
  if (ws_bytes < bitffn::decode_stack_workspace_bytes(d_model, d_ff, T, top_k)) return MOE_ENOSPC;
  const bitffn::StackDims D{d_model, d_ff, n_experts, top_k, T};
  return hip_status(bitffn::launch_decode_stack(D, n_layers, layers, x, ws, stream));
}

int moe_decode_misses(const moe_layer* H, const float* x, int T, const int32_t* idx,
                      const int32_t* slot, const float* w, const int32_t* host_slot_of_expert,
                      int max_rank, float* y, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_decode_misses_phases(H, x, T, idx, slot, w, host_slot_of_expert, max_rank, y, ws,
                                  ws_bytes, MOE_MISSES_READ | MOE_MISSES_JOIN, stream);
}

int moe_decode_misses_phases(const moe_layer* H, const float* x, int T, const int32_t* idx,
                             const int32_t* slot, const float* w,
                             const int32_t* host_slot_of_expert, int max_rank, float* y, void* ws,
                             size_t ws_bytes, int phases, hipStream_t stream) {
  const int st = check_layer(H);
  if (st != MOE_OK) return st;
  if (H->shared_slot != -1) return MOE_EINVAL;
  if (T < 1 || T > MOE_MAX_DECODE_T || T * H->top_k > MOE_MAX_DECODE_PAIRS) return MOE_EINVAL;
  if (max_rank < 0 || max_rank > H->top_k) return MOE_EINVAL;
  if (phases < 1 || phases > (MOE_MISSES_READ | MOE_MISSES_JOIN)) return MOE_EINVAL;
  const bool read = (phases & MOE_MISSES_READ) != 0, join = (phases & MOE_MISSES_JOIN) != 0;
  if (!idx || !slot || !host_slot_of_expert || !ws || (read && !x) || (join && (!w || !y)))
    return MOE_EINVAL;
  if (x && y && static_cast<const void*>(x) == static_cast<const void*>(y)) return MOE_EINVAL;
  if ((x && !aligned16(x)) || !aligned16(idx) || !aligned16(slot) || (w && !aligned16(w)) ||
      !aligned16(host_slot_of_expert) || (y && !aligned16(y)))
    return MOE_EALIGN;
  if (!aligned256(ws)) return MOE_EALIGN;
  if (ws_bytes < bitffn::decode_workspace_bytes(H->d_model, H->d_ff, T, H->top_k))
    return MOE_ENOSPC;
  // The pool must be memory this device can address: pinned host memory
  // (its device-side address is used) or device memory.
  const void* pool_dev = nullptr;
  if (!device_address(H->pool, &pool_dev)) return MOE_EINVAL;
  if (max_rank == 0) return MOE_OK;   // no miss can run
  return hip_status(bitffn::launch_decode_misses(*H, pool_dev, x, T, idx, slot, w,
                                                 host_slot_of_expert, max_rank, y, ws, stream,
                                                 phases));
}

int moe_cache_count(const int32_t* idx, int n_pairs, int E, uint32_t* counts,
                    hipStream_t stream) {
  if (n_pairs < 0 || n_pairs >= (1 << 24) || E < 1 || E > MOE_MAX_EXPERTS) return MOE_EINVAL;
  if (n_pairs == 0) return MOE_OK;
  if (!idx || !counts) return MOE_EINVAL;
  if (!aligned16(idx) || !aligned16(counts)) return MOE_EALIGN;
  return hip_status(bitffn::launch_cache_count(idx, n_pairs, E, counts, stream));
}

int moe_cache_plan(uint32_t* counts, int E, int32_t* slot_of_expert, int32_t* expert_of_slot,
                   int n_slots, int shared_slot, const int32_t* host_slot_of_expert,
                   int host_n_slots, int max_swaps, int decay_shift, int32_t* swaps,
                   int32_t* n_swaps, hipStream_t stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS) return MOE_EINVAL;
  if (n_slots < 1 || n_slots > MOE_MAX_CACHE_SLOTS) return MOE_EINVAL;
  if (shared_slot < -1 || shared_slot >= n_slots || host_n_slots < 0) return MOE_EINVAL;
  if (max_swaps < 1 || max_swaps > MOE_MAX_EXPERTS || decay_shift < 0 || decay_shift > 31)
    return MOE_EINVAL;
  if (!counts || !slot_of_expert || !expert_of_slot || !host_slot_of_expert || !swaps || !n_swaps)
    return MOE_EINVAL;
  if (!aligned16(counts) || !aligned16(slot_of_expert) || !aligned16(expert_of_slot) ||
      !aligned16(host_slot_of_expert) || !aligned16(swaps) || !aligned16(n_swaps))
    return MOE_EALIGN;
  return hip_status(bitffn::launch_cache_plan(counts, E, slot_of_expert, expert_of_slot, n_slots,
                                              shared_slot, host_slot_of_expert, host_n_slots,
                                              max_swaps, decay_shift, swaps, n_swaps, stream));
}

int moe_cache_fill(const moe_layer* L, const moe_layer* H, const int32_t* swaps,
                   const int32_t* n_swaps, int max_swaps, hipStream_t stream) {
  int st = check_layer(L);
  if (st != MOE_OK) return st;
  st = check_layer(H);
  if (st != MOE_OK) return st;
  if (L->fmt != H->fmt || L->d_model != H->d_model || L->d_ff != H->d_ff) return MOE_EFORMAT;
  if (max_swaps < 1 || max_swaps > MOE_MAX_EXPERTS) return MOE_EINVAL;
  if (!swaps || !n_swaps) return MOE_EINVAL;
  if (!aligned16(swaps) || !aligned16(n_swaps)) return MOE_EALIGN;
  const void* host_dev = nullptr;
  if (!device_address(H->pool, &host_dev)) return MOE_EINVAL;
  return hip_status(bitffn::launch_cache_fill(host_dev, H->n_slots, const_cast<void*>(L->pool),
                                              L->n_slots, L->slot_bytes, swaps, n_swaps,
                                              max_swaps, stream));
}

int moe_cache_commit(int32_t* slot_of_expert, int E, const int32_t* swaps,
                     const int32_t* n_swaps, int max_swaps, hipStream_t stream) {
  if (E < 1 || E > MOE_MAX_EXPERTS || max_swaps < 1 || max_swaps > MOE_MAX_EXPERTS)
    return MOE_EINVAL;
  if (!slot_of_expert || !swaps || !n_swaps) return MOE_EINVAL;
  if (!aligned16(slot_of_expert) || !aligned16(swaps) || !aligned16(n_swaps)) return MOE_EALIGN;
  return hip_status(bitffn::launch_cache_commit(slot_of_expert, E, swaps, n_swaps, max_swaps,
                                                stream));
}

int moe_stage_layer(const moe_layer* C, const int32_t* slot_of_expert, const moe_layer* H,
                    const int32_t* host_slot_of_expert, void* staging, size_t staging_bytes,
                    hipStream_t stream) {
  int st = check_layer(C);
  if (st != MOE_OK) return st;
  st = check_layer(H);
  if (st != MOE_OK) return st;
  if (C->fmt != H->fmt || C->d_model != H->d_model || C->d_ff != H->d_ff) return MOE_EFORMAT;
  if (C->n_experts != H->n_experts) return MOE_EINVAL;
  if (!slot_of_expert || !host_slot_of_expert || !staging) return MOE_EINVAL;
  if (!aligned256(staging)) return MOE_EALIGN;
  const int E = C->n_experts;
  for (int e = 0; e < E; ++e) {   // every expert needs a source
    const int cs = slot_of_expert[e], hs = host_slot_of_expert[e];
    const bool in_cache = cs >= 0 && cs < C->n_slots && cs != C->shared_slot;
    const bool in_host = hs >= 0 && hs < H->n_slots;
    if (!in_cache && (cs >= 0 || !in_host)) return MOE_EINVAL;
  }
  if (staging_bytes < static_cast<size_t>(E + 1) * static_cast<size_t>(C->slot_bytes))
    return MOE_ENOSPC;
  const void* host_dev = nullptr;
  if (!device_address(H->pool, &host_dev)) return MOE_EINVAL;
  return hip_status(bitffn::launch_stage_layer(*C, slot_of_expert, H->pool, host_slot_of_expert,
                                               staging, stream));
}

size_t moe_prefill_workspace_bytes(const moe_layer* L, int T) {
  if (check_layer(L) != MOE_OK || T < 1 || T > 65536) return 0;
  return bitffn::prefill_workspace_bytes(L->d_model, L->d_ff, T, L->top_k, L->n_experts);
}

int moe_expert_ffn_prefill(const moe_layer* L, const uint16_t* x_bf16, int T, const int32_t* idx,
                           const int32_t* slot, float* out_pairs, int32_t* pair_pos,
                           int32_t* expert_offsets, float* out_shared, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  const int st = check_layer(L);
  if (st != MOE_OK) return st;
  if (T < 1 || T > 65536) return MOE_EINVAL;
  if (L->d_model % 128 != 0 || L->d_ff % 64 != 0) return MOE_EINVAL;
  // the GEMMs address x and h through 32-bit buffer offsets
  if (static_cast<int64_t>(T) * (L->top_k + 1) * L->d_ff * 2 >= (int64_t{1} << 32)) return MOE_EINVAL;
  if (!x_bf16 || !idx || !slot || !out_pairs || !pair_pos || !expert_offsets || !ws)
    return MOE_EINVAL;
  if (out_shared && L->shared_slot < 0) return MOE_EINVAL;
  if (!aligned16(x_bf16) || !aligned16(idx) || !aligned16(slot) || !aligned16(out_pairs) ||
      !aligned16(pair_pos) || !aligned16(expert_offsets) || (out_shared && !aligned16(out_shared)))
    return MOE_EALIGN;
  if (!aligned256(ws)) return MOE_EALIGN;
  if (ws_bytes < bitffn::prefill_workspace_bytes(L->d_model, L->d_ff, T, L->top_k, L->n_experts))
    return MOE_ENOSPC;
  return hip_status(bitffn::launch_prefill(*L, x_bf16, T, idx, slot, out_pairs, pair_pos,
                                           expert_offsets, out_shared, ws, stream));
}

int moe_combine(const void* x, int x_dtype, int T, int d, int k, const float* rows,
                const int32_t* pair_pos, const float* w, const float* shared, float* y,
                hipStream_t stream) {
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_EINVAL;
  if (T < 0 || d < 4 || d % 4 != 0 || k < 0 || k > MOE_MAX_TOPK) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !y) return MOE_EINVAL;
  if (k > 0 && (!rows || !pair_pos || !w)) return MOE_EINVAL;
  if (x_dtype == MOE_DTYPE_BF16 && static_cast<const void*>(y) == x) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(y) || (rows && !aligned16(rows)) ||
      (pair_pos && !aligned16(pair_pos)) || (w && !aligned16(w)) || (shared && !aligned16(shared)))
    return MOE_EALIGN;
  return hip_status(
      bitffn::launch_combine(x, x_dtype, T, d, k, rows, pair_pos, w, shared, y, stream));
}

}  // extern "C"
