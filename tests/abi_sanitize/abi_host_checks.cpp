// Host-side argument checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_abi_sanitized.py
// builds and runs it).  Every call below fails its checks before any HIP
// call, so no device is needed and no pointer given here is dereferenced
// except the host-side ones: the layer structs, the layer array of
// moe_decode_stack and the slot tables of moe_stage_layer.  The size checks
// of those two calls come after their walks over the array and the tables,
// so the calls that fail only on size read every entry; the sanitizers
// report any read past them, and any undefined arithmetic in the checks.
// Prints "abi host checks: N passed, 0 failed" and exits 0, or names each
// failing check and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "bitffn_moe.h"

namespace {

int g_checks = 0, g_failed = 0;

void expect(long long got, long long want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    ++g_failed;
    std::printf("FAILED line %d: %s returned %lld, expected %lld\n", line, what, got, want);
  }
}
#define EXPECT(call, want) expect(static_cast<long long>(call), static_cast<long long>(want), #call, __LINE__)

// Fake device addresses: never dereferenced, since every call fails first.
constexpr uintptr_t kFake = 0x7F0000000000ull;
template <typename T = void>
T* fp(uintptr_t off = 0) {
  return reinterpret_cast<T*>(kFake + off);
}
const hipStream_t s0 = nullptr;

int64_t sb(int fmt, int d, int f) { return moe_slot_bytes(fmt, d, f); }

moe_layer layer(int d = 2048, int f = 768, int E = 512, int k = 10, int fmt = MOE_FMT_Q2SM,
                int n_slots = 513, int shared = 512) {
  moe_layer L;
  std::memset(&L, 0, sizeof L);
  L.d_model = d;
  L.d_ff = f;
  L.n_experts = E;
  L.top_k = k;
  L.fmt = fmt;
  L.n_slots = n_slots;
  L.shared_slot = shared;
  L.reserved = 0;
  L.slot_bytes = sb(fmt, d, f);
  L.pool = fp();
  return L;
}

void version_and_sizes() {
  EXPECT(moe_abi_version(), MOE_ABI_VERSION);
  for (int st = -6; st <= 0; ++st) EXPECT(moe_status_str(st) != nullptr, 1);
  EXPECT(std::strcmp(moe_status_str(-99), "unknown status"), 0);
  EXPECT(moe_last_hip_error(), 0);
  EXPECT(sb(4, 256, 128), MOE_EFORMAT);
  EXPECT(sb(MOE_FMT_Q2SM, 96, 128), MOE_EINVAL);
  EXPECT(sb(MOE_FMT_Q2SM, 4096, 128), MOE_EINVAL);
  EXPECT(sb(MOE_FMT_Q2SM, 256, 80), MOE_EINVAL);
  EXPECT(sb(MOE_FMT_Q2SM, 256, 8192), MOE_EINVAL);
  EXPECT(sb(MOE_FMT_Q2SM, 2048, 768) > 0, 1);
  EXPECT(sb(MOE_FMT_Q2SM, 2048, 768) % 256, 0);
  // extreme arguments: no overflow in the size arithmetic
  EXPECT(sb(MOE_FMT_Q3G, 1 << 30, 1 << 30), MOE_EINVAL);
  EXPECT(sb(MOE_FMT_Q3G, -64, 32), MOE_EINVAL);
  EXPECT(moe_lookup_workspace_bytes(4, 10, 512), 0);
  EXPECT(moe_lookup_workspace_bytes(8192, 10, 512) > 0, 1);
  EXPECT(moe_lookup_workspace_bytes(1 << 30, 64, 1024) >= 0, 1);
  EXPECT(moe_lookup_workspace_bytes(-1, 10, 512), 0);
}

void router() {
  auto call = [&](int T, int d, int E, float* x, uint16_t* w, float* out) {
    return moe_router_logits(x, T, d, w, E, out, s0);
  };
  float* x = fp<float>();
  uint16_t* w = fp<uint16_t>(1 << 20);
  float* out = fp<float>(1 << 24);
  EXPECT(call(0, 2048, 512, x, w, out), MOE_EINVAL);
  EXPECT(call(5, 2048, 512, x, w, out), MOE_EINVAL);
  EXPECT(call(1, 96, 512, x, w, out), MOE_EINVAL);
  EXPECT(call(1, 4096, 512, x, w, out), MOE_EINVAL);
  EXPECT(call(1, 1 << 30, 512, x, w, out), MOE_EINVAL);
  EXPECT(call(1, 2048, 0, x, w, out), MOE_EINVAL);
  EXPECT(call(1, 2048, 2000, x, w, out), MOE_EINVAL);
  EXPECT(call(1, 2048, 512, nullptr, w, out), MOE_EINVAL);
  EXPECT(call(1, 2048, 512, x, nullptr, out), MOE_EINVAL);
  EXPECT(call(1, 2048, 512, x, w, nullptr), MOE_EINVAL);
  EXPECT(call(1, 2048, 512, x, w, x), MOE_EINVAL);
  EXPECT(call(1, 2048, 512, fp<float>(4), w, out), MOE_EALIGN);
  EXPECT(call(1, 2048, 512, x, fp<uint16_t>((1 << 20) + 8), out), MOE_EALIGN);
  EXPECT(call(1, 2048, 512, x, w, fp<float>((1 << 24) + 4)), MOE_EALIGN);
}

void route_and_lookup() {
  EXPECT(moe_route_topk(fp<float>(), 1, 0, 1, fp<int32_t>(), fp<float>(), s0), MOE_EINVAL);
  EXPECT(moe_route_topk(fp<float>(), 1, 2000, 4, fp<int32_t>(), fp<float>(), s0), MOE_EINVAL);
  EXPECT(moe_route_topk(fp<float>(), 1, 64, 65, fp<int32_t>(), fp<float>(), s0), MOE_EINVAL);
  EXPECT(moe_route_topk(fp<float>(), 1, 8, 9, fp<int32_t>(), fp<float>(), s0), MOE_EINVAL);
  EXPECT(moe_route_topk(fp<float>(), -1, 64, 4, fp<int32_t>(), fp<float>(), s0), MOE_EINVAL);
  EXPECT(moe_route_topk(fp<float>(), 1 << 30, 64, 4, fp<int32_t>(), fp<float>(), s0), MOE_EINVAL);
  EXPECT(moe_route_topk(nullptr, 1, 64, 4, fp<int32_t>(), fp<float>(), s0), MOE_EINVAL);
  EXPECT(moe_route_topk(fp<float>(4), 1, 64, 4, fp<int32_t>(), fp<float>(), s0), MOE_EALIGN);
  EXPECT(moe_route_topk(nullptr, 0, 64, 4, nullptr, nullptr, s0), MOE_OK);

  int32_t* p = fp<int32_t>();
  EXPECT(moe_cache_lookup(p, 1, 0, p, 64, p, p, p, p, nullptr, 0, s0), MOE_EINVAL);
  EXPECT(moe_cache_lookup(nullptr, 1, 4, p, 64, p, p, p, p, nullptr, 0, s0), MOE_EINVAL);
  EXPECT(moe_cache_lookup(fp<int32_t>(8), 1, 4, p, 64, p, p, p, p, nullptr, 0, s0), MOE_EALIGN);
  const size_t need = moe_lookup_workspace_bytes(8192, 10, 512);
  EXPECT(moe_cache_lookup(p, 8192, 10, p, 512, p, p, p, p, nullptr, 0, s0), MOE_EINVAL);
  EXPECT(moe_cache_lookup(p, 8192, 10, p, 512, p, p, p, p, fp(), need - 1, s0), MOE_ENOSPC);
}

void decode() {
  moe_layer L = layer();
  const size_t need = moe_decode_workspace_bytes(&L, 1);
  EXPECT(need > 0, 1);
  EXPECT(moe_decode_workspace_bytes(&L, 5), 0);
  EXPECT(moe_decode_workspace_bytes(nullptr, 1), 0);
  auto ffn = [&](const moe_layer& l, int T, size_t ws, float* y) {
    return moe_expert_ffn_decode(&l, fp<float>(), T, fp<int32_t>(), fp<int32_t>(), fp<float>(), y,
                                 fp(), ws, s0);
  };
  float* y = fp<float>(1 << 20);
  EXPECT(ffn(L, 1, need - 1, y), MOE_ENOSPC);
  EXPECT(ffn(L, 5, need, y), MOE_EINVAL);
  EXPECT(ffn(layer(2048, 768, 512, 20), 4, need, y), MOE_EINVAL);
  EXPECT(ffn(L, 1, need, fp<float>()), MOE_EINVAL);
  EXPECT(ffn(layer(2048, 768, 512, 10, 7), 1, need, y), MOE_EFORMAT);
  moe_layer b = layer();
  b.slot_bytes = 12345;
  EXPECT(ffn(b, 1, need, y), MOE_EFORMAT);
  b = layer();
  b.pool = fp(16);
  EXPECT(ffn(b, 1, need, y), MOE_EALIGN);
  EXPECT(ffn(layer(2048, 768, 512, 10, MOE_FMT_Q2SM, 513, 513), 1, need, y), MOE_EINVAL);
  b = layer();
  b.reserved = 1;
  EXPECT(ffn(b, 1, need, y), MOE_EINVAL);
  EXPECT(ffn(layer(2048, 768, 512, 0), 1, need, y), MOE_EINVAL);
  EXPECT(ffn(layer(3000), 1, need, y), MOE_EINVAL);
  b = layer();
  b.n_slots = 0;
  EXPECT(ffn(b, 1, need, y), MOE_EINVAL);

  // the one-call layer and its allocation-free variant: same checks, and the
  // latter refuses sizes past its scratch before any HIP call
  auto lay = [&](const moe_layer& l, int T, float* x, float* yy, void* ws, size_t nb) {
    return moe_decode_layer(&l, x, T, fp<float>(1 << 16), fp<int32_t>(1 << 17), fp<int32_t>(1 << 18),
                            fp<float>(1 << 19), fp<int32_t>(1 << 21), fp<int32_t>(1 << 22),
                            nullptr, fp<int32_t>(1 << 23), yy, ws, nb, s0);
  };
  auto noalloc = [&](const moe_layer& l, int T, float* x, float* yy) {
    return moe_decode_layer_noalloc(&l, x, T, fp<float>(1 << 16), fp<int32_t>(1 << 17),
                                    fp<int32_t>(1 << 18), fp<float>(1 << 19), fp<int32_t>(1 << 21),
                                    fp<int32_t>(1 << 22), nullptr, fp<int32_t>(1 << 23), yy, s0);
  };
  EXPECT(lay(L, 1, fp<float>(), y, fp(), need - 1), MOE_ENOSPC);
  EXPECT(lay(L, 1, fp<float>(), y, nullptr, need), MOE_EINVAL);
  EXPECT(lay(L, 1, fp<float>(), y, fp(16), need), MOE_EALIGN);
  EXPECT(lay(L, 1, nullptr, y, fp(), need), MOE_EINVAL);
  EXPECT(lay(L, 1, fp<float>(), fp<float>(), fp(), need), MOE_EINVAL);
  EXPECT(lay(L, 0, fp<float>(), y, fp(), need), MOE_EINVAL);
  EXPECT(noalloc(L, 0, fp<float>(), y), MOE_EINVAL);
  EXPECT(noalloc(L, 5, fp<float>(), y), MOE_EINVAL);
  EXPECT(noalloc(L, 1, nullptr, y), MOE_EINVAL);
  EXPECT(noalloc(L, 1, fp<float>(), fp<float>()), MOE_EINVAL);
  EXPECT(noalloc(L, 1, fp<float>(4), y), MOE_EALIGN);
  EXPECT(noalloc(layer(2048, 4096, 1024, 16), 4, fp<float>(), y), MOE_ENOSPC);
}

void prefill_and_combine() {
  moe_layer L = layer();
  const size_t need = moe_prefill_workspace_bytes(&L, 8192);
  EXPECT(need > 0, 1);
  auto call = [&](const moe_layer& l, int T, size_t ws, float* shared) {
    return moe_expert_ffn_prefill(&l, fp<uint16_t>(), T, fp<int32_t>(), fp<int32_t>(), fp<float>(),
                                  fp<int32_t>(), fp<int32_t>(), shared, fp(), ws, s0);
  };
  EXPECT(call(L, 8192, need - 1, fp<float>()), MOE_ENOSPC);
  EXPECT(call(L, 0, need, fp<float>()), MOE_EINVAL);
  EXPECT(call(L, 70000, need, fp<float>()), MOE_EINVAL);
  EXPECT(call(layer(2048, 768, 512, 10, MOE_FMT_Q2SM, 513, -1), 8192, need, fp<float>()),
         MOE_EINVAL);
  EXPECT(call(layer(64), 8192, size_t{1} << 40, fp<float>()), MOE_EINVAL);
  EXPECT(call(layer(2048, 4096, 512, 64), 65536, size_t{1} << 40, fp<float>()), MOE_EINVAL);
  EXPECT(moe_prefill_workspace_bytes(&L, 1 << 30) == 0 || moe_prefill_workspace_bytes(&L, 1 << 30) > need, 1);

  float* f = fp<float>();
  int32_t* i = fp<int32_t>();
  EXPECT(moe_combine(f, 3, 1, 64, 4, f, i, f, nullptr, fp<float>(1 << 12), s0), MOE_EINVAL);
  EXPECT(moe_combine(f, 0, 1, 66, 4, f, i, f, nullptr, fp<float>(1 << 12), s0), MOE_EINVAL);
  EXPECT(moe_combine(f, 0, 1, 64, 4, nullptr, i, f, nullptr, fp<float>(1 << 12), s0), MOE_EINVAL);
  EXPECT(moe_combine(f, 1, 1, 64, 4, f, i, f, nullptr, f, s0), MOE_EINVAL);
  EXPECT(moe_combine(fp<float>(4), 0, 1, 64, 4, f, i, f, nullptr, fp<float>(1 << 12), s0), MOE_EALIGN);
  EXPECT(moe_combine(nullptr, 0, 0, 64, 4, nullptr, nullptr, nullptr, nullptr, nullptr, s0), MOE_OK);
}

void misses() {
  moe_layer H = layer(2048, 768, 512, 10, MOE_FMT_Q2SM, 512, -1);
  const size_t need = moe_decode_workspace_bytes(&H, 1);
  auto call = [&](const moe_layer& h, int T, int max_rank, size_t ws, float* y) {
    return moe_decode_misses(&h, fp<float>(), T, fp<int32_t>(), fp<int32_t>(), fp<float>(),
                             fp<int32_t>(), max_rank, y, fp(), ws, s0);
  };
  float* y = fp<float>(1 << 20);
  EXPECT(call(layer(2048, 768, 512, 10, MOE_FMT_Q2SM, 512, 3), 1, 10, need, y), MOE_EINVAL);
  EXPECT(call(H, 1, 11, need, y), MOE_EINVAL);
  EXPECT(call(H, 1, -1, need, y), MOE_EINVAL);
  EXPECT(call(H, 5, 10, need, y), MOE_EINVAL);
  EXPECT(call(H, 1, 10, need - 1, y), MOE_ENOSPC);
  EXPECT(call(H, 1, 10, need, fp<float>()), MOE_EINVAL);
  EXPECT(call(layer(2048, 768, 512, 10, 9, 512, -1), 1, 10, need, y), MOE_EFORMAT);
  auto phases = [&](int ph, float* x, float* yy, float* w) {
    return moe_decode_misses_phases(&H, x, 1, fp<int32_t>(), fp<int32_t>(), w, fp<int32_t>(), 10,
                                    yy, fp(), need, ph, s0);
  };
  EXPECT(phases(0, fp<float>(), y, fp<float>(1 << 21)), MOE_EINVAL);
  EXPECT(phases(4, fp<float>(), y, fp<float>(1 << 21)), MOE_EINVAL);
  EXPECT(phases(MOE_MISSES_READ, nullptr, y, fp<float>(1 << 21)), MOE_EINVAL);
  EXPECT(phases(MOE_MISSES_JOIN, fp<float>(), nullptr, fp<float>(1 << 21)), MOE_EINVAL);
  EXPECT(phases(MOE_MISSES_JOIN, fp<float>(), y, nullptr), MOE_EINVAL);
  EXPECT(phases(MOE_MISSES_READ | MOE_MISSES_JOIN, fp<float>(), fp<float>(), fp<float>(1 << 21)),
         MOE_EINVAL);
  EXPECT(phases(MOE_MISSES_JOIN, nullptr, fp<float>(8), fp<float>(1 << 21)), MOE_EALIGN);
}

void layer_tiers() {
  moe_layer L = layer();
  moe_layer H = layer(2048, 768, 512, 10, MOE_FMT_Q2SM, 512, -1);
  const size_t need = moe_decode_workspace_bytes(&L, 1);
  auto call = [&](const moe_layer& l, const moe_layer& h, int T, int max_rank, const int32_t* host,
                  float* yy, void* ws, size_t nb) {
    return moe_decode_layer_tiers(&l, &h, host, max_rank, fp<float>(), T, fp<float>(1 << 16),
                                  fp<int32_t>(1 << 17), fp<int32_t>(1 << 18), fp<float>(1 << 19),
                                  fp<int32_t>(1 << 21), fp<int32_t>(1 << 22), nullptr,
                                  fp<int32_t>(1 << 23), yy, ws, nb, s0);
  };
  float* y = fp<float>(1 << 20);
  const int32_t* hs = fp<int32_t>(1 << 24);
  EXPECT(call(L, H, 1, 10, hs, y, fp(), need - 1), MOE_ENOSPC);
  EXPECT(call(L, H, 1, 10, hs, y, nullptr, need), MOE_EINVAL);
  EXPECT(call(L, H, 1, 10, hs, y, fp(16), need), MOE_EALIGN);
  EXPECT(call(L, H, 1, 10, nullptr, y, fp(), need), MOE_EINVAL);
  EXPECT(call(L, H, 1, 10, fp<int32_t>(4), y, fp(), need), MOE_EALIGN);
  EXPECT(call(L, H, 1, 11, hs, y, fp(), need), MOE_EINVAL);
  EXPECT(call(L, H, 1, -1, hs, y, fp(), need), MOE_EINVAL);
  EXPECT(call(L, H, 5, 10, hs, y, fp(), need), MOE_EINVAL);
  EXPECT(call(L, H, 1, 10, hs, fp<float>(), fp(), need), MOE_EINVAL);
  EXPECT(call(L, layer(2048, 768, 512, 10, MOE_FMT_Q2SM, 512, 3), 1, 10, hs, y, fp(), need),
         MOE_EINVAL);
  EXPECT(call(L, layer(2048, 768, 512, 8, MOE_FMT_Q2SM, 512, -1), 1, 10, hs, y, fp(), need),
         MOE_EINVAL);
  EXPECT(call(L, layer(2048, 768, 256, 10, MOE_FMT_Q2SM, 512, -1), 1, 10, hs, y, fp(), need),
         MOE_EINVAL);
  EXPECT(call(L, layer(2048, 768, 512, 10, MOE_FMT_Q3G, 512, -1), 1, 10, hs, y, fp(), need),
         MOE_EINVAL);
  moe_layer hb = H;
  hb.pool = fp(16);
  EXPECT(call(L, hb, 1, 10, hs, y, fp(), need), MOE_EALIGN);
  EXPECT(call(layer(2048, 768, 512, 10, 9), H, 1, 10, hs, y, fp(), need), MOE_EFORMAT);
}

void cache_policy() {
  int32_t* p = fp<int32_t>();
  uint32_t* c = fp<uint32_t>();
  EXPECT(moe_cache_count(p, 10, 0, c, s0), MOE_EINVAL);
  EXPECT(moe_cache_count(p, 10, 2000, c, s0), MOE_EINVAL);
  EXPECT(moe_cache_count(p, -1, 512, c, s0), MOE_EINVAL);
  EXPECT(moe_cache_count(nullptr, 0, 512, nullptr, s0), MOE_OK);
  EXPECT(moe_cache_count(fp<int32_t>(4), 10, 512, c, s0), MOE_EALIGN);
  auto plan = [&](int E, int n_slots, int shared, int max_swaps, int shift, const int32_t* hs,
                  int32_t* swaps) {
    return moe_cache_plan(c, E, p, p, n_slots, shared, hs, 512, max_swaps, shift, swaps, p, s0);
  };
  EXPECT(plan(0, 95, 94, 8, 1, p, p), MOE_EINVAL);
  EXPECT(plan(512, 0, 94, 8, 1, p, p), MOE_EINVAL);
  EXPECT(plan(512, 5000, 94, 8, 1, p, p), MOE_EINVAL);
  EXPECT(plan(512, 95, 95, 8, 1, p, p), MOE_EINVAL);
  EXPECT(plan(512, 95, 94, 0, 1, p, p), MOE_EINVAL);
  EXPECT(plan(512, 95, 94, 1025, 1, p, p), MOE_EINVAL);
  EXPECT(plan(512, 95, 94, 8, 32, p, p), MOE_EINVAL);
  EXPECT(plan(512, 95, 94, 8, -1, p, p), MOE_EINVAL);
  EXPECT(plan(512, 95, 94, 8, 1, nullptr, p), MOE_EINVAL);
  EXPECT(plan(512, 95, 94, 8, 1, p, fp<int32_t>(8)), MOE_EALIGN);

  moe_layer L = layer();
  moe_layer H = layer(2048, 768, 512, 10, MOE_FMT_Q2SM, 512, -1);
  moe_layer H1 = layer(2048, 768, 512, 10, MOE_FMT_Q2S, 512, -1);
  EXPECT(moe_cache_fill(&L, &H1, p, p, 8, s0), MOE_EFORMAT);
  EXPECT(moe_cache_fill(&L, &H, p, p, 0, s0), MOE_EINVAL);
  EXPECT(moe_cache_fill(&L, &H, fp<int32_t>(4), p, 8, s0), MOE_EALIGN);
  moe_layer Hm = H;
  Hm.pool = fp(16);
  EXPECT(moe_cache_fill(&L, &Hm, p, p, 8, s0), MOE_EALIGN);
  EXPECT(moe_cache_fill(nullptr, &H, p, p, 8, s0), MOE_EINVAL);
  EXPECT(moe_cache_commit(p, 0, p, p, 8, s0), MOE_EINVAL);
  EXPECT(moe_cache_commit(p, 512, p, p, 0, s0), MOE_EINVAL);
  EXPECT(moe_cache_commit(p, 512, nullptr, p, 8, s0), MOE_EINVAL);
}

void stage() {
  const int E = 512;
  const moe_layer C = layer(2048, 768, E, 10, MOE_FMT_Q2SM, 95, 94);
  const moe_layer H = layer(2048, 768, E, 10, MOE_FMT_Q2SM, 512, -1);
  // host arrays of exactly n_experts entries: a read past them is reported
  std::vector<int32_t> soe(E, -1), hs(E);
  for (int e = 0; e < 94; ++e) soe[e] = e;
  for (int e = 0; e < E; ++e) hs[e] = e;
  const size_t nbytes = static_cast<size_t>(E + 1) * static_cast<size_t>(sb(MOE_FMT_Q2SM, 2048, 768));
  auto call = [&](const moe_layer& c, const moe_layer& h, const std::vector<int32_t>& s,
                  const std::vector<int32_t>& hh, void* st, size_t nb) {
    return moe_stage_layer(&c, s.data(), &h, hh.data(), st, nb, s0);
  };
  EXPECT(call(C, H, soe, hs, fp(), nbytes - 256), MOE_ENOSPC);   // walks both tables
  EXPECT(call(C, H, soe, hs, fp(16), nbytes), MOE_EALIGN);
  EXPECT(call(C, layer(2048, 768, 500, 10, MOE_FMT_Q2SM, 512, -1), soe, hs, fp(), nbytes),
         MOE_EINVAL);
  EXPECT(call(C, layer(2048, 768, E, 10, MOE_FMT_Q2S, 512, -1), soe, hs, fp(), nbytes),
         MOE_EFORMAT);
  std::vector<int32_t> bad = hs;
  bad[200] = -1;   // expert 200 in neither tier
  EXPECT(call(C, H, soe, bad, fp(), nbytes), MOE_EINVAL);
  bad = hs;
  bad[E - 1] = 512;   // host slot out of range, in the last entry
  EXPECT(call(C, H, soe, bad, fp(), nbytes), MOE_EINVAL);
  std::vector<int32_t> bsoe = soe;
  bsoe[300] = 94;   // the shared slot is no expert's home
  bad = hs;
  bad[300] = -1;
  EXPECT(call(C, H, bsoe, bad, fp(), nbytes), MOE_EINVAL);
}

void stack() {
  const int64_t b = sb(MOE_FMT_Q2SM, 2048, 768);
  auto sl = [&]() {
    moe_stack_layer l;
    std::memset(&l, 0, sizeof l);
    l.pool = fp();
    l.slot_bytes = b;
    l.n_slots = 513;
    l.fmt = MOE_FMT_Q2SM;
    l.shared_slot = 512;
    l.slot_of_expert = fp<int32_t>(1 << 16);
    l.logits = fp<float>(1 << 17);
    l.y = fp<float>(1 << 18);
    return l;
  };
  const size_t need = moe_decode_stack_workspace_bytes(2048, 768, 512, 10, 1);
  EXPECT(need > 0, 1);
  EXPECT(moe_decode_stack_workspace_bytes(2048, 768, 512, 10, 5), 0);
  EXPECT(moe_decode_stack_workspace_bytes(2048, 768, 512, 20, 4), 0);
  EXPECT(moe_decode_stack_workspace_bytes(2048, 768, 1025, 10, 1), 0);
  EXPECT(moe_decode_stack_workspace_bytes(-2048, 768, 512, 10, 1), 0);
  auto call = [&](std::vector<moe_stack_layer> ls, int n, int T, int k, float* x, void* ws,
                  size_t nb) {
    return moe_decode_stack(2048, 768, 512, k, T, n, ls.data(), x, ws, nb, s0);
  };
  float* x = fp<float>(1 << 21);
  void* ws = fp(1 << 22);
  moe_stack_layer first = sl(), last = sl();
  first.y = nullptr;
  std::vector<moe_stack_layer> ok = {first, last};
  EXPECT(call(ok, 0, 1, 10, x, ws, need), MOE_EINVAL);
  EXPECT(call(ok, -3, 1, 10, x, ws, need), MOE_EINVAL);
  EXPECT(call(ok, 2, 5, 10, x, ws, need), MOE_EINVAL);
  EXPECT(call(ok, 2, 4, 20, x, ws, need), MOE_EINVAL);
  EXPECT(call(ok, 2, 1, 10, x, ws, need - 1), MOE_ENOSPC);   // walks both layers
  EXPECT(call(ok, 2, 1, 10, x, fp((1 << 22) + 16), need), MOE_EALIGN);
  EXPECT(call(ok, 2, 1, 10, nullptr, ws, need), MOE_EINVAL);
  EXPECT(call({sl(), first}, 2, 1, 10, x, ws, need), MOE_EINVAL);   // last y required
  auto with = [&](auto edit) {
    moe_stack_layer l = sl();
    edit(l);
    return std::vector<moe_stack_layer>{first, l};
  };
  EXPECT(call(with([](moe_stack_layer& l) { l.fmt = 7; }), 2, 1, 10, x, ws, need), MOE_EFORMAT);
  EXPECT(call(with([&](moe_stack_layer& l) { l.slot_bytes = b + 256; }), 2, 1, 10, x, ws, need),
         MOE_EFORMAT);
  EXPECT(call(with([](moe_stack_layer& l) { l.reserved = 1; }), 2, 1, 10, x, ws, need), MOE_EINVAL);
  EXPECT(call(with([](moe_stack_layer& l) { l.shared_slot = 513; }), 2, 1, 10, x, ws, need),
         MOE_EINVAL);
  EXPECT(call(with([](moe_stack_layer& l) { l.logits = nullptr; }), 2, 1, 10, x, ws, need),
         MOE_EINVAL);
  EXPECT(call(with([](moe_stack_layer& l) { l.idx = fp<int32_t>(1 << 19); }), 2, 1, 10, x, ws, need),
         MOE_EINVAL);
  EXPECT(call(with([](moe_stack_layer& l) { l.n_miss = fp<int32_t>(1 << 19); }), 2, 1, 10, x, ws,
              need),
         MOE_EINVAL);
  EXPECT(call(with([](moe_stack_layer& l) { l.pool = fp(16); }), 2, 1, 10, x, ws, need), MOE_EALIGN);
  EXPECT(call(with([](moe_stack_layer& l) { l.addend = fp<float>((1 << 19) + 4); }), 2, 1, 10, x, ws,
              need),
         MOE_EALIGN);
  EXPECT(call(with([](moe_stack_layer& l) { l.y = fp<float>(1 << 21); }), 2, 1, 10, x, ws, need),
         MOE_EINVAL);
}

}  // namespace

int main() {
  version_and_sizes();
  router();
  route_and_lookup();
  decode();
  prefill_and_combine();
  misses();
  layer_tiers();
  cache_policy();
  stage();
  stack();
  std::printf("abi host checks: %d passed, %d failed\n", g_checks - g_failed, g_failed);
  return g_failed == 0 ? 0 : 1;
}
