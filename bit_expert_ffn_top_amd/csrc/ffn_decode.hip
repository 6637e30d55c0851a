// Decode / verify layer for T <= 4 tokens.
//
// 1. plan (one wavefront): the distinct resident experts chosen by the T
//    tokens, in order of first appearance over (t, i), each with the mask of
//    tokens that chose it; pair_pos[t*k+i] = u*T + t for a hit, -1 for a miss.
//    The shared expert takes the fixed union index T*k.
// 2. gate/up (one wavefront per (union expert, 8 rows of h)): each lane owns
//    64 consecutive columns of G, i.e. two 32-weight blocks, so a row of
//    d_model columns is spread over d_model/64 lanes and one 16-byte load per
//    lane per row fetches the codes.  All the workgroup's weight bytes are
//    loaded before any arithmetic; each token that chose the expert then
//    reuses them from registers.  Row sums are reduced across the lanes of
//    the row; gate and up rows of the same h index sit in neighbouring lane
//    groups, so h = silu(g) * u needs one more exchange.
// 3. down (one wavefront per (union expert, 64 output rows)): each lane owns
//    BD consecutive blocks of a D row (d_ff / (32 BD) lanes per row) and
//    keeps its slice of h in registers for all the rows it visits.
// 4. combine: y = x + sum_i w * o_i + o_shared in k-slot order.
// Every weight byte of a chosen expert is read once per call, however many
// of the T tokens chose it.
#include "moe_internal.h"

namespace bitffn {
namespace {

constexpr int kPlanUSlot = 1;
constexpr int kPlanUMask = 1 + MOE_MAX_DECODE_PAIRS;
constexpr int kPlanPairPos = 1 + 2 * MOE_MAX_DECODE_PAIRS;
constexpr int kPlanInts = 1 + 3 * MOE_MAX_DECODE_PAIRS;

__global__ __launch_bounds__(64) void decode_plan_kernel(const int32_t* __restrict__ slot, int T,
                                                         int k, int32_t* __restrict__ plan) {
  const int p = threadIdx.x;
  const int n = T * k;
  const int s = p < n ? slot[p] : -1;
  const bool hit = s >= 0;
  bool first = hit;
  for (int q = 0; q < n; ++q) {
    const int sq = __shfl(s, q, 64);
    if (q < p && sq == s) first = false;
  }
  const uint64_t fm = __ballot(first);
  const int u_first = __popcll(fm & ((1ull << p) - 1ull));
  int my_u = -1;
  uint32_t mask = 0;
  for (int q = 0; q < n; ++q) {
    const int sq = __shfl(s, q, 64);
    const int uq = __shfl(u_first, q, 64);
    const bool fq = (fm >> q) & 1ull;
    if (hit && sq == s) {
      mask |= 1u << (q / k);
      if (fq) my_u = uq;
    }
  }
  if (first) {
    plan[kPlanUSlot + u_first] = s;
    plan[kPlanUMask + u_first] = static_cast<int32_t>(mask);
  }
  if (p < n) plan[kPlanPairPos + p] = hit ? my_u * T + p / k : -1;
  if (p == 0) plan[0] = __popcll(fm);
}

__device__ __forceinline__ bool decode_union_member(const int32_t* plan, int u, int T, int k,
                                                    int shared_slot, int& slot, uint32_t& mask) {
  if (u == T * k) {
    if (shared_slot < 0) return false;
    slot = shared_slot;
    mask = (1u << T) - 1u;
    return true;
  }
  if (u >= plan[0]) return false;
  slot = plan[kPlanUSlot + u];
  mask = static_cast<uint32_t>(plan[kPlanUMask + u]);
  return true;
}

// NLPR: lanes per G row (= d_model / 64).
template <int FMT, int NLPR>
__global__ __launch_bounds__(64) void decode_gateup_kernel(
    const uint8_t* __restrict__ pool, int64_t slot_bytes, Planes GP, int d, int f, int T, int k,
    int shared_slot, const float* __restrict__ x, const int32_t* __restrict__ plan,
    float* __restrict__ hbuf) {
  constexpr int RPW = 64 / NLPR;                 // rows per wave iteration
  constexpr int J = RPW <= 16 ? 8 : RPW / 2;     // h indices per workgroup
  constexpr int NIT = 2 * J / RPW;               // iterations
  int sl;
  uint32_t mask;
  const int u = blockIdx.y;
  if (!decode_union_member(plan, u, T, k, shared_slot, sl, mask)) return;
  const uint8_t* base = pool + static_cast<int64_t>(sl) * slot_bytes;
  const int lane = threadIdx.x;
  const int c = lane % NLPR;
  const int rr = lane / NLPR;
  const int nb = d / 32;
  const int j0 = blockIdx.x * J;

  uint4 cw[NIT];
  uint32_t sc[NIT], mn[NIT];
  uint2 hw[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int64_t r = 2 * j0 + it * RPW + rr;
    const int64_t blk = r * nb + 2 * c;
    cw[it] = *reinterpret_cast<const uint4*>(base + GP.codes + blk * 8);
    sc[it] = *reinterpret_cast<const uint32_t*>(base + GP.scale + blk * 2);
    if (FMT == MOE_FMT_Q2SM) mn[it] = *reinterpret_cast<const uint32_t*>(base + GP.min + blk * 2);
    if (FMT == MOE_FMT_Q3G) hw[it] = *reinterpret_cast<const uint2*>(base + GP.hi + blk * 4);
  }

  for (int t = 0; t < T; ++t) {
    if (!((mask >> t) & 1u)) continue;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      opaque(cw[it]);
      opaque(sc[it]);
      if (FMT == MOE_FMT_Q2SM) opaque(mn[it]);
      if (FMT == MOE_FMT_Q3G) opaque(hw[it]);
    }
    float xv[64];
    const float4* xp = reinterpret_cast<const float4*>(x + static_cast<int64_t>(t) * d + 64 * c);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const float4 v = xp[q];
      xv[4 * q] = v.x;
      xv[4 * q + 1] = v.y;
      xv[4 * q + 2] = v.z;
      xv[4 * q + 3] = v.w;
    }
    float xs0 = 0.0f, xs1 = 0.0f;
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      xs0 += xv[q];
      xs1 += xv[32 + q];
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const float s0 = half_bits_to_float(sc[it] & 0xFFFFu);
      const float s1 = half_bits_to_float(sc[it] >> 16);
      float m0 = 0.0f, m1 = 0.0f;
      if (FMT == MOE_FMT_Q2SM) {
        m0 = half_bits_to_float(mn[it] & 0xFFFFu);
        m1 = half_bits_to_float(mn[it] >> 16);
      }
      const uint32_t h0 = FMT == MOE_FMT_Q3G ? hw[it].x : 0u;
      const uint32_t h1 = FMT == MOE_FMT_Q3G ? hw[it].y : 0u;
      float part = block_dot<FMT>(cw[it].x, cw[it].y, h0, s0, m0, xv, xs0);
      part += block_dot<FMT>(cw[it].z, cw[it].w, h1, s1, m1, xv + 32, xs1);
#pragma unroll
      for (int o = NLPR / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
      const float other = __shfl_xor(part, NLPR, 64);
      if ((rr & 1) == 0 && c == 0) {
        const int j = j0 + (it * RPW + rr) / 2;
        hbuf[(static_cast<int64_t>(u) * T + t) * f + j] = silu(part) * other;
      }
    }
  }
}

// BD: blocks per lane, LD: lanes per D row (BD * LD = d_ff / 32).
template <int FMT, int BD, int LD>
__global__ __launch_bounds__(64) void decode_down_kernel(
    const uint8_t* __restrict__ pool, int64_t slot_bytes, Planes DP, int d, int f, int T, int k,
    int shared_slot, const int32_t* __restrict__ plan, const float* __restrict__ hbuf,
    float* __restrict__ obuf) {
  constexpr int RPI = 64 / LD;   // rows per iteration
  constexpr int ROWS = 64;       // rows per workgroup
  constexpr int NIT = ROWS / RPI;
  int sl;
  uint32_t mask;
  const int u = blockIdx.y;
  if (!decode_union_member(plan, u, T, k, shared_slot, sl, mask)) return;
  const uint8_t* base = pool + static_cast<int64_t>(sl) * slot_bytes;
  const int lane = threadIdx.x;
  const int c = lane % LD;
  const int rr = lane / LD;
  const int nb = f / 32;
  const int r0 = blockIdx.x * ROWS;

  uint2 cw[NIT][BD];
  uint32_t sc[NIT][BD], mn[NIT][BD], hw[NIT][BD];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int64_t r = r0 + it * RPI + rr;
#pragma unroll
    for (int b = 0; b < BD; ++b) {
      const int64_t blk = r * nb + c * BD + b;
      cw[it][b] = *reinterpret_cast<const uint2*>(base + DP.codes + blk * 8);
      sc[it][b] = *reinterpret_cast<const uint16_t*>(base + DP.scale + blk * 2);
      if (FMT == MOE_FMT_Q2SM) mn[it][b] = *reinterpret_cast<const uint16_t*>(base + DP.min + blk * 2);
      if (FMT == MOE_FMT_Q3G) hw[it][b] = *reinterpret_cast<const uint32_t*>(base + DP.hi + blk * 4);
    }
  }

  for (int t = 0; t < T; ++t) {
    if (!((mask >> t) & 1u)) continue;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
#pragma unroll
      for (int b = 0; b < BD; ++b) {
        opaque(cw[it][b]);
        opaque(sc[it][b]);
        if (FMT == MOE_FMT_Q2SM) opaque(mn[it][b]);
        if (FMT == MOE_FMT_Q3G) opaque(hw[it][b]);
      }
    }
    float hv[BD * 32];
    const float4* hp = reinterpret_cast<const float4*>(
        hbuf + (static_cast<int64_t>(u) * T + t) * f + c * BD * 32);
#pragma unroll
    for (int q = 0; q < BD * 8; ++q) {
      const float4 v = hp[q];
      hv[4 * q] = v.x;
      hv[4 * q + 1] = v.y;
      hv[4 * q + 2] = v.z;
      hv[4 * q + 3] = v.w;
    }
    float hs[BD];
#pragma unroll
    for (int b = 0; b < BD; ++b) {
      float a = 0.0f;
#pragma unroll
      for (int q = 0; q < 32; ++q) a += hv[32 * b + q];
      hs[b] = a;
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float part = 0.0f;
#pragma unroll
      for (int b = 0; b < BD; ++b) {
        const float s = half_bits_to_float(sc[it][b]);
        const float m = FMT == MOE_FMT_Q2SM ? half_bits_to_float(mn[it][b]) : 0.0f;
        part += block_dot<FMT>(cw[it][b].x, cw[it][b].y, FMT == MOE_FMT_Q3G ? hw[it][b] : 0u, s, m,
                               hv + 32 * b, hs[b]);
      }
#pragma unroll
      for (int o = LD / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
      if (c == 0) {
        const int64_t r = r0 + it * RPI + rr;
        obuf[(static_cast<int64_t>(u) * T + t) * d + r] = part;
      }
    }
  }
}

struct DecodeWs {
  int32_t* plan;
  float* h;
  float* o;
};

DecodeWs decode_ws(void* ws, int d, int f, int T, int k) {
  char* p = static_cast<char*>(ws);
  DecodeWs w;
  w.plan = reinterpret_cast<int32_t*>(p);
  p += align256(kPlanInts * 4);
  w.h = reinterpret_cast<float*>(p);
  p += align256(static_cast<int64_t>(T * k + 1) * T * f * 4);
  w.o = reinterpret_cast<float*>(p);
  return w;
}

template <int FMT, int NLPR>
hipError_t launch_gateup_f(const moe_layer& L, const SlotLayout& lay, int T, const float* x,
                           const DecodeWs& w, hipStream_t s) {
  constexpr int RPW = 64 / NLPR;
  constexpr int J = RPW <= 16 ? 8 : RPW / 2;
  const dim3 grid(L.d_ff / J, L.top_k * T + 1);
  decode_gateup_kernel<FMT, NLPR><<<grid, 64, 0, s>>>(
      static_cast<const uint8_t*>(L.pool), L.slot_bytes, lay.G, L.d_model, L.d_ff, T, L.top_k,
      L.shared_slot, x, w.plan, w.h);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gateup(const moe_layer& L, const SlotLayout& lay, int T, const float* x,
                         const DecodeWs& w, hipStream_t s) {
  switch (L.d_model / 64) {
    case 1: return launch_gateup_f<FMT, 1>(L, lay, T, x, w, s);
    case 2: return launch_gateup_f<FMT, 2>(L, lay, T, x, w, s);
    case 4: return launch_gateup_f<FMT, 4>(L, lay, T, x, w, s);
    case 8: return launch_gateup_f<FMT, 8>(L, lay, T, x, w, s);
    case 16: return launch_gateup_f<FMT, 16>(L, lay, T, x, w, s);
    case 32: return launch_gateup_f<FMT, 32>(L, lay, T, x, w, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT, int BD, int LD>
hipError_t launch_down_f(const moe_layer& L, const SlotLayout& lay, int T, const DecodeWs& w,
                         hipStream_t s) {
  const dim3 grid(L.d_model / 64, L.top_k * T + 1);
  decode_down_kernel<FMT, BD, LD><<<grid, 64, 0, s>>>(
      static_cast<const uint8_t*>(L.pool), L.slot_bytes, lay.D, L.d_model, L.d_ff, T, L.top_k,
      L.shared_slot, w.plan, w.h, w.o);
  return hipGetLastError();
}

template <int FMT, int BD>
hipError_t launch_down_bd(const moe_layer& L, const SlotLayout& lay, int T, const DecodeWs& w,
                          hipStream_t s) {
  switch (L.d_ff / 32 / BD) {
    case 1: return launch_down_f<FMT, BD, 1>(L, lay, T, w, s);
    case 2: return launch_down_f<FMT, BD, 2>(L, lay, T, w, s);
    case 4: return launch_down_f<FMT, BD, 4>(L, lay, T, w, s);
    case 8: return launch_down_f<FMT, BD, 8>(L, lay, T, w, s);
    case 16: return launch_down_f<FMT, BD, 16>(L, lay, T, w, s);
    case 32: return launch_down_f<FMT, BD, 32>(L, lay, T, w, s);
    case 64: return launch_down_f<FMT, BD, 64>(L, lay, T, w, s);
    default: return hipErrorInvalidValue;
  }
}

template <int FMT>
hipError_t launch_down(const moe_layer& L, const SlotLayout& lay, int T, const DecodeWs& w,
                       hipStream_t s) {
  const int nb = L.d_ff / 32;
  if (nb % 3 == 0) return launch_down_bd<FMT, 3>(L, lay, T, w, s);
  return launch_down_bd<FMT, 1>(L, lay, T, w, s);
}

template <int FMT>
hipError_t launch_decode_fmt(const moe_layer& L, const float* x, int T, const float* wts,
                             float* y, const DecodeWs& w, hipStream_t s) {
  const SlotLayout lay = slot_layout(L.fmt, L.d_model, L.d_ff);
  hipError_t e = launch_gateup<FMT>(L, lay, T, x, w, s);
  if (e != hipSuccess) return e;
  e = launch_down<FMT>(L, lay, T, w, s);
  if (e != hipSuccess) return e;
  const float* shared = L.shared_slot >= 0
                            ? w.o + static_cast<int64_t>(T) * L.top_k * T * L.d_model
                            : nullptr;
  return launch_combine(x, MOE_DTYPE_F32, T, L.d_model, L.top_k, w.o, w.plan + kPlanPairPos,
                        wts, shared, y, s);
}

}  // namespace

size_t decode_workspace_bytes(int d, int f, int T, int k) {
  return static_cast<size_t>(align256(kPlanInts * 4) +
                             align256(static_cast<int64_t>(T * k + 1) * T * f * 4) +
                             align256(static_cast<int64_t>(T * k + 1) * T * d * 4));
}

hipError_t launch_decode(const moe_layer& L, const float* x, int T, const int32_t* idx,
                         const int32_t* slot, const float* w, float* y, void* ws,
                         hipStream_t s) {
  (void)idx;
  const DecodeWs dw = decode_ws(ws, L.d_model, L.d_ff, T, L.top_k);
  decode_plan_kernel<<<1, 64, 0, s>>>(slot, T, L.top_k, dw.plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (L.fmt) {
    case MOE_FMT_Q2S: return launch_decode_fmt<MOE_FMT_Q2S>(L, x, T, w, y, dw, s);
    case MOE_FMT_Q2SM: return launch_decode_fmt<MOE_FMT_Q2SM>(L, x, T, w, y, dw, s);
    case MOE_FMT_Q3G: return launch_decode_fmt<MOE_FMT_Q3G>(L, x, T, w, y, dw, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bitffn
