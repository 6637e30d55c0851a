// Decode / verify layer for T <= 4 tokens: two kernels, no waiting between
// workgroups inside a kernel.
//
// Union of experts.  Union member u < T*k is pair u = t*k+i if its slot is a
// hit and no earlier pair names the same slot; it serves every token that
// chose that slot.  Member T*k is the shared expert (all tokens).  Every
// member's packed bytes are read once per call.
//
// 1. ffn kernel, one workgroup of 16 wavefronts per (member u, slice js of 32
//    h indices).  Gate/up: the slice owns G rows 64js..64js+63 (gate and up
//    rows of h indices 32js..32js+31); lane l streams row 64js+l, so every
//    load of a wavefront reads one 1 KiB unit of 64 consecutive rows, and the
//    activation x is the same for all lanes (scalar operands).  The 16
//    wavefronts split the d_model columns in interleaved 64-column units;
//    their row sums meet in LDS in a fixed order, and h = silu(g) * u is
//    formed for the 32 h indices.
//    Down, split over d_ff: the same workgroup multiplies its 32 h values into
//    block column js of D (all d_model rows) and stores that partial product.
//    Weight bytes of both parts are loaded before any arithmetic.
// 2. combine kernel: y[t] = x[t] + sum_i w[t,i] * (sum over slices of the
//    partials of member u(t,i)) + (same for the shared member), slices summed
//    in a fixed tree, terms in k-slot order, shared last.
// Arithmetic per block: codes become fp16 pairs (c + q) by mask-and-OR with
// an exponent, each multiplied into fp32 by v_fma_mix; the block's offset sum
// and scale/min are applied once per block.
//
// Modes of the ffn kernel: the pair slots given (moe_expert_ffn_decode), the
// routing done inside every workgroup (moe_decode_layer), the missed pairs
// only, with their slots in a second pool such as pinned host memory
// (moe_decode_misses, whose combine adds into y), or the routing inside with
// the combine's weighted sum accumulated into buffers by atomic adds
// (moe_decode_layer_acc, whose y a later call finishes).
#include "moe_internal.h"
#include "route_device.h"

namespace bitffn {
namespace {

// Expert weights are streamed once per call: nontemporal loads keep them out
// of the caches that x, the logits and the slot table are read through.
typedef uint32_t nu4 __attribute__((ext_vector_type(4)));
typedef uint32_t nu2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 stream_u4(const uint8_t* p) {
  const nu4 v = __builtin_nontemporal_load(reinterpret_cast<const nu4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 stream_u2(const uint8_t* p) {
  const nu2 v = __builtin_nontemporal_load(reinterpret_cast<const nu2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t stream_u32(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t stream_u16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

// x is read-only for the whole kernel: reading it through the constant address
// space lets its wavefront-uniform loads become scalar loads.
typedef const __attribute__((address_space(4))) float cfloat;

constexpr int KA_THREADS = 1024;
constexpr int KA_WAVES = KA_THREADS / 64;
constexpr int SLICE = 32;          // h indices per workgroup
constexpr int MAX_DROWS = 2048 / KA_THREADS;   // D rows per thread: d_model <= 2048
static_assert(2048 / 64 <= 4 * KA_WAVES, "G units per wavefront above 4");

// What selects the union members' slots.
enum FfnMode {
  kPairs = 0,   // the pair slots given by the caller
  kRoute = 1,   // routing done in the kernel (top-k, slot table)
  kMiss = 2,    // missed pairs only, their slots in a second pool (host tier)
  kAcc = 3,     // routing in the kernel; weighted terms added into acc buffers
};

// Accumulation buffers of the kAcc mode: term contributions of slice js go to
// buffer js % ACC_BUFS, so that an element takes (members x slices / ACC_BUFS)
// atomic adds instead of one add per slice and member.
constexpr int ACC_BUFS = 8;

struct FfnArgs {
  const uint8_t* pool;
  int64_t slot_bytes;
  Planes G, D;
  int d, f, T, k, shared_slot;
  const int32_t* slot;
  float* part;  // [T][k+1][f/32][d]: term i of token t, the shared expert at i = k
  // fused routing only: inputs, and the routing outputs written by
  // workgroup (0, 0)
  const float* logits;          // [T][E]
  const int32_t* table;         // slot_of_expert [E]
  int E;
  int32_t* o_idx;               // [T][k]
  float* o_w;                   // [T][k]
  int32_t* o_slot;              // [T][k]
  int32_t* o_miss_expert;       // [<= T*k]
  int32_t* o_miss_pair;         // [T*k] or null
  int32_t* o_n_miss;            // [2]
  // miss mode only: the pairs' experts; `table` is then the host tier's
  // slot of each expert (entries outside [0, n_slots) count as absent), and
  // a miss of k-slot i runs only if i < max_rank
  const int32_t* idx;           // [T][k]
  int max_rank, n_slots;
  // kAcc only: acc_out [ACC_BUFS][T][d] (zero on entry) receives the weighted
  // terms; acc_clear (same shape, optional) is set to zero; if prev_acc is
  // given, prev_y = prev_x + sum over its buffers (the previous call's y)
  float* acc_out;
  float* acc_clear;
  const float* prev_x;
  const float* prev_acc;
  float* prev_y;
};

// One row job of the kAcc side workgroups (and of the finish kernel): row r
// < n_zero of `zero` ([n_zero][d]) is set to zero; row n_zero + t is
// y[t] = x[t] + acc[0][t] + ... + acc[ACC_BUFS-1][t], added in that order.
// 1024 threads, two values each (d <= 2048, d even).
__device__ __forceinline__ void acc_row_job(int r, int n_zero, float* __restrict__ zero, int T,
                                            int d, const float* __restrict__ x,
                                            const float* __restrict__ acc,
                                            float* __restrict__ y) {
  const int c = 2 * static_cast<int>(threadIdx.x);
  if (c >= d) return;
  if (r < n_zero) {
    *reinterpret_cast<float2*>(zero + static_cast<int64_t>(r) * d + c) = make_float2(0.0f, 0.0f);
    return;
  }
  const int t = r - n_zero;
  const int64_t o = static_cast<int64_t>(t) * d + c;
  float2 v[ACC_BUFS + 1];
  v[0] = *reinterpret_cast<const float2*>(x + o);
#pragma unroll
  for (int b = 0; b < ACC_BUFS; ++b)
    v[b + 1] = *reinterpret_cast<const float2*>(acc + static_cast<int64_t>(b) * T * d + o);
  float2 sum = v[0];
#pragma unroll
  for (int b = 1; b <= ACC_BUFS; ++b) {
    sum.x += v[b].x;
    sum.y += v[b].y;
  }
  *reinterpret_cast<float2*>(y + o) = sum;
}

// y = x + the ACC_BUFS buffers of acc, token t per workgroup.
__global__ __launch_bounds__(KA_THREADS) void acc_finish_kernel(const float* __restrict__ x,
                                                                const float* __restrict__ acc,
                                                                int T, int d,
                                                                float* __restrict__ y) {
  acc_row_job(blockIdx.x, 0, nullptr, T, d, x, acc, y);
}

// Survivors of the first top-k level in the fused kernel: T * ceil(E/64) * k
// <= 16 * (T * k) <= 16 * 64.
constexpr int kFusedCand = (MOE_MAX_EXPERTS / 64) * MOE_MAX_DECODE_PAIRS;
static_assert(MOE_MAX_EXPERTS <= KA_THREADS, "one slot-table entry per thread");
static_assert(MOE_MAX_DECODE_T * (MOE_MAX_EXPERTS / 64) <= 4 * KA_WAVES,
              "logit groups per wavefront above 4");

// Union member u: its slot, the mask of tokens it serves, and `same`, the
// mask of pairs naming that slot (all of them for the shared expert, whose
// term is i = k).  `sp` is the slot of pair `lane` (-1 for lanes >= T*k;
// T*k <= 64), so the test is a lane read and a ballot; the result is uniform
// across the wavefront.
__device__ __forceinline__ bool union_member(int sp, int T, int k, int shared_slot, int u,
                                             int& s, uint32_t& mask, uint64_t& same) {
  const int n = T * k;
  if (u == n) {
    if (shared_slot < 0) return false;
    s = shared_slot;
    mask = (1u << T) - 1u;
    same = 0;
    return true;
  }
  s = __builtin_amdgcn_readlane(sp, u);
  if (s < 0) return false;
  same = __ballot(sp == s);
  if (same & ((1ull << u) - 1ull)) return false;   // an earlier pair names this slot
  const uint64_t kmask = k >= 64 ? ~0ull : (1ull << k) - 1ull;
  mask = 0;
  for (int t = 0; t < T; ++t)
    if ((same >> (t * k)) & kmask) mask |= 1u << t;
  return true;
}

// k-slot of the member's pair in token t (a token names a slot at most once)
__device__ __forceinline__ int member_term(uint64_t same, int t, int k, bool shared) {
  return shared ? k : __builtin_ctzll(same >> (t * k));
}

// value of v in lane `src` (uniform result)
__device__ __forceinline__ float lane_value(float v, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), src));
}

template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// sum over each row of 16 lanes, complete in every lane of the row
__device__ __forceinline__ float row16_sum(float v) {
  v = add_dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v = add_dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v = add_dpp<0x124>(v);   // row_ror:4
  return add_dpp<0x128>(v);   // row_ror:8
}

// sum over the wavefront (uniform result): rows of 16 by DPP, then the four
// row sums in the fixed order (r0 + r1) + (r2 + r3)
__device__ __forceinline__ float wave_total(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// UPW: G units (2 blocks) per wavefront, ceil(d_model / 64 / KA_WAVES); wavefront
// w takes units w, w + KA_WAVES, ...  d_model <= 2048.
// MODE kRoute: the workgroup first routes the T tokens itself (top-k over the
// logits, slots from the slot table held in LDS) instead of reading the pair
// slots; workgroups of the shared expert skip routing.  MODE kMiss: a pair's
// slot is its expert's slot in the host tier if the pair missed the GPU
// cache and its rank is below the limit, else none; there is no shared
// member.  MODE kAcc: routing as kRoute; each served token's term, times its
// routing weight (1 for the shared expert), is added into buffer js % ACC_BUFS
// of acc_out; the last row of workgroups (u = T*k + 1) only does the row jobs
// of acc_row_job (clearing acc_clear, finishing prev_y).
template <int FMT, int UPW, int MODE>
__global__ __launch_bounds__(KA_THREADS) void decode_ffn_kernel(FfnArgs a,
                                                                const float* __restrict__ x) {
  constexpr bool ROUTE = MODE == kRoute || MODE == kAcc;
  const int js = blockIdx.x;
  const int u = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int d = a.d;
  const int n = a.T * a.k;
  if (MODE == kAcc && u == n + 1) {   // side workgroups: row jobs only
    const int n_zero = a.acc_clear ? ACC_BUFS * a.T : 0;
    const int jobs = n_zero + (a.prev_acc ? a.T : 0);
    for (int r = js; r < jobs; r += gridDim.x)
      acc_row_job(r, n_zero, a.acc_clear, a.T, d, a.prev_x, a.prev_acc, a.prev_y);
    return;
  }
  int sp = -1;   // slot of pair `lane`
  if (MODE == kPairs) sp = lane < n ? a.slot[lane] : -1;
  if (MODE == kMiss) {
    const int p = min(lane, n - 1);
    const int gpu_slot = a.slot[p];
    const int e = min(max(a.idx[p], 0), a.E - 1);
    const int hs = a.table[e];
    sp = lane < n && gpu_slot < 0 && p % a.k < a.max_rank && hs < a.n_slots ? hs : -1;
  }

  // Every load below is unconditional, with indices clamped into range (the
  // surplus values are never used), so the compiler can count outstanding
  // loads and wait for each group alone.  Order: the pair slots, x (needed
  // first, by the block sums), G units in the order they are used, then D.
  float2 xv[MOE_MAX_DECODE_T];
  const int ex = min(2 * tid, d - 2);
#pragma unroll
  for (int t = 0; t < MOE_MAX_DECODE_T; ++t) {
    const int tt = min(t, a.T - 1);
    xv[t] = *reinterpret_cast<const float2*>(x + static_cast<int64_t>(tt) * d + ex);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep the issue order

  __shared__ float s_wt[MOE_MAX_DECODE_PAIRS];   // kAcc: routing weight of pair t*k + i
  if (ROUTE && u < n) {   // uniform per workgroup
    __shared__ uint64_t s_grp[KA_WAVES * 64];
    __shared__ uint64_t s_cand[kFusedCand];
    __shared__ uint64_t s_top[MOE_MAX_DECODE_PAIRS];
    __shared__ int32_t s_table[MOE_MAX_EXPERTS];
    float lg[4];
    topk_load<4>(a.logits, a.T, a.E, lg);
    const int tv = a.table[min(tid, a.E - 1)];
    topk_select<4>(lg, a.T, a.E, a.k, TopkLds{s_grp, s_cand, s_top}, [&] {
      if (tid < a.E) s_table[tid] = tv;
    });
    const int e = lane < n ? key_expert(s_top[lane]) : 0;
    sp = lane < n ? s_table[e] : -1;
    if (MODE == kAcc && wave < a.T) {   // this workgroup's own routing weights
      int id;
      float wt;
      topk_softmax_lane(s_top + wave * a.k, a.k, lane, id, wt);
      if (lane < a.k) s_wt[wave * a.k + lane] = wt;
    }
    if (u == 0 && js == 0) {   // routing outputs
      if (wave < a.T) {
        int id;
        float wt;
        topk_softmax_lane(s_top + wave * a.k, a.k, lane, id, wt);
        if (lane < a.k) {
          a.o_idx[wave * a.k + lane] = id;
          a.o_w[wave * a.k + lane] = wt;
          a.o_slot[wave * a.k + lane] = s_table[id];
        }
      }
      if (wave == KA_WAVES - 1)
        wave_miss_lists(lane, n, e, sp, a.o_miss_expert, a.o_miss_pair, a.o_n_miss);
    }
  }

  int s;
  uint32_t mask;
  uint64_t same;
  if (!union_member(sp, a.T, a.k, a.shared_slot, u, s, mask, same)) return;
  const uint8_t* __restrict__ base = a.pool + static_cast<int64_t>(s) * a.slot_bytes;
  const int64_t R = 2 * static_cast<int64_t>(a.f);   // G rows
  const int64_t grow = 2 * SLICE * js + lane;        // this lane's G row
  const int nu = d / 64;

  // ---- loads: G units of this wavefront, then D block column js ----
  uint4 gc[UPW];
  uint32_t gs[UPW], gm[UPW];
  uint2 gh[UPW];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int64_t unit = static_cast<int64_t>(min(wave + KA_WAVES * i, nu - 1)) * R + grow;
    gc[i] = stream_u4(base + a.G.codes + unit * 16);
    gs[i] = stream_u32(base + a.G.scale + unit * 4);
    if (FMT == MOE_FMT_Q2SM) gm[i] = stream_u32(base + a.G.min + unit * 4);
    if (FMT == MOE_FMT_Q3G) gh[i] = stream_u2(base + a.G.hi + unit * 8);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int ndr = (d - tid + KA_THREADS - 1) / KA_THREADS;   // D rows of this thread
  uint2 dc[MAX_DROWS];
  uint32_t ds[MAX_DROWS], dm[MAX_DROWS], dh[MAX_DROWS];
#pragma unroll
  for (int i = 0; i < MAX_DROWS; ++i) {
    const int64_t unit = static_cast<int64_t>(js) * d + min(tid + KA_THREADS * i, d - 1);
    dc[i] = stream_u2(base + a.D.codes + unit * 8);
    ds[i] = stream_u16(base + a.D.scale + unit * 2);
    if (FMT == MOE_FMT_Q2SM) dm[i] = stream_u16(base + a.D.min + unit * 2);
    if (FMT == MOE_FMT_Q3G) dh[i] = stream_u32(base + a.D.hi + unit * 4);
  }

  __shared__ float red[KA_WAVES][64];
  __shared__ float2 bsum[MOE_MAX_DECODE_T][2048 / 32];   // per block of x: (sum, offset constant)
  __shared__ __attribute__((aligned(16))) float hsh[SLICE];
  __shared__ float hsum[2];

  // per-block sums of x (sum, offset constant) for every served token: each
  // thread adds two neighbouring values, the 16 threads of a block reduce by
  // DPP rotations within their row of 16 lanes; lane 0 of the row stores
  // (computed for all token slots, stored for served ones: no branch for
  // the compiler to sink the x loads into)
  const float cw0 = block_offset_weight<FMT>(ex & 31), cw1 = block_offset_weight<FMT>((ex & 31) + 1);
#pragma unroll
  for (int t = 0; t < MOE_MAX_DECODE_T; ++t) {
    const float sx = row16_sum(xv[t].x + xv[t].y);
    const float sc = row16_sum(fmaf(cw1, xv[t].y, cw0 * xv[t].x));
    if (((mask >> t) & 1u) && (tid & 15) == 0 && 2 * tid < d)
      bsum[t][tid >> 4] = make_float2(sx, block_const<FMT>(sx, sc));
  }
  __syncthreads();

  const int nslices = a.f / SLICE;
  // one served token: gate/up, SiLU gating, partial down product
  auto token_pass = [&](int t) {
    const float* __restrict__ xt = x + static_cast<int64_t>(t) * d;

    // gate/up rows: partial sums over this wavefront's units (x as scalar
    // operands)
    float row = 0.0f;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int c = wave + KA_WAVES * i;
      if (c < nu) {
        const cfloat* xw = (const cfloat*)(xt + 64 * c);
        const float2 s0 = bsum[t][2 * c], s1 = bsum[t][2 * c + 1];
        const uint32_t hw0 = FMT == MOE_FMT_Q3G ? gh[i].x : 0u;
        const uint32_t hw1 = FMT == MOE_FMT_Q3G ? gh[i].y : 0u;
        const uint32_t m = FMT == MOE_FMT_Q2SM ? gm[i] : 0u;
        const float acc0 = block_acc<FMT>(gc[i].x, gc[i].y, hw0, xw, 0);
        row = block_finish<FMT>(row, acc0, s0.y, s0.x, gs[i], m);
        const float acc1 = block_acc<FMT>(gc[i].z, gc[i].w, hw1, xw, 32);
        row = block_finish<FMT>(row, acc1, s1.y, s1.x, gs[i] >> 16, m >> 16);
      }
    }
    red[wave][lane] = row;
    __syncthreads();
    if (wave == 0) {
      float rs = red[0][lane];
#pragma unroll
      for (int w = 1; w < KA_WAVES; ++w) rs += red[w][lane];
      // up row 2j+1 sits in the lane after gate row 2j (DPP quad_perm [1,0,3,2])
      const float up = __builtin_bit_cast(
          float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, rs), 0xB1, 0xF, 0xF, false));
      const float hv = silu(rs) * up;                       // valid in even lanes
      const int j = lane >> 1;
      const bool even = (lane & 1) == 0;
      if (even) hsh[j] = hv;
      const float hx = wave_total(even ? hv : 0.0f);
      const float hc = wave_total(even ? block_offset_weight<FMT>(j) * hv : 0.0f);
      if (lane == 0) {
        hsum[0] = hx;
        hsum[1] = block_const<FMT>(hx, hc);
      }
    }
    __syncthreads();

    // down: this slice's block column of D, all rows.  h is read from LDS
    // (same address in every lane) 16 values at a time, each half applied to
    // every row of the thread before the next half is read.
    const float HX = hsum[0], HK = hsum[1];
    const int term = member_term(same, t, a.k, u == n);
    float* __restrict__ out =
        MODE == kAcc ? a.acc_out + (static_cast<int64_t>(js % ACC_BUFS) * a.T + t) * d
                     : a.part + ((static_cast<int64_t>(t) * (a.k + 1) + term) * nslices + js) * d;
    const float wterm = MODE == kAcc ? (u == n ? 1.0f : s_wt[t * a.k + term]) : 1.0f;
    float a0[MAX_DROWS], a1[MAX_DROWS];
#pragma unroll
    for (int i = 0; i < MAX_DROWS; ++i) a0[i] = a1[i] = 0.0f;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float hv[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = reinterpret_cast<const float4*>(hsh)[4 * half + q];
        hv[4 * q] = v.x;
        hv[4 * q + 1] = v.y;
        hv[4 * q + 2] = v.z;
        hv[4 * q + 3] = v.w;
      }
#pragma unroll
      for (int i = 0; i < MAX_DROWS; ++i) {
        if (i < ndr) {
          const uint32_t w = half ? dc[i].y : dc[i].x;
          if (FMT == MOE_FMT_Q3G) {
            if (half == 0) dot16_q3<0>(w, dh[i], hv, 0, a0[i], a1[i]);
            else dot16_q3<-1>(w, dh[i], hv, 0, a0[i], a1[i]);
          } else {
            dot16_q2(w, hv, 0, a0[i], a1[i]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < MAX_DROWS; ++i) {
      if (i < ndr) {
        const float v = block_finish<FMT>(0.0f, a0[i] + a1[i], HK, HX, ds[i],
                                          FMT == MOE_FMT_Q2SM ? dm[i] : 0u);
        if (MODE == kAcc)
          unsafeAtomicAdd(out + tid + KA_THREADS * i, wterm * v);
        else
          out[tid + KA_THREADS * i] = v;
      }
    }
    __syncthreads();
  };

  // The first served token runs outside the loop, so its arithmetic waits for
  // each load group alone (entering a loop makes the compiler wait for every
  // outstanding load).  Later tokens reuse the weights held in registers;
  // marking them as rewritten each iteration keeps the compiler from hoisting
  // per-token decode work out of the loop.
  token_pass(__builtin_ctz(mask));
  for (uint32_t rest = mask & (mask - 1u); rest != 0u; rest &= rest - 1u) {
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      opaque(gc[i]);
      opaque(gs[i]);
      if (FMT == MOE_FMT_Q2SM) opaque(gm[i]);
      if (FMT == MOE_FMT_Q3G) opaque(gh[i]);
    }
#pragma unroll
    for (int i = 0; i < MAX_DROWS; ++i) {
      opaque(dc[i]);
      opaque(ds[i]);
      if (FMT == MOE_FMT_Q2SM) opaque(dm[i]);
      if (FMT == MOE_FMT_Q3G) opaque(dh[i]);
    }
    token_pass(__builtin_ctz(rest));
  }
}

// y = x + sum_{i: slot >= 0} w_i * P(t, i) + P(t, k), P(t, i) = sum over
// slices of term i's partials (P(t, k): the shared expert, if any).
// MISS: y += sum_{i in the miss set} w_i * P(t, i), the miss set as the ffn
// kernel's miss mode selects it; no shared term.
// Workgroup: 32 rows (128 bytes of a partial row: whole memory lines), one
// wavefront per term (terms i, i+16, ...); lane = (row r, slice group g of
// 2), group g sums its half of the slices in order, the two group sums meet
// as g0 + g1, and wavefront 0 adds the terms in k-slot order, shared last.
// No load depends on another: x, w, the pair slots and every partial are
// requested up front (terms without partials are loaded and not used; in the
// miss mode the terms outside the miss set are skipped, since the reads of
// that mode cross the host link).
constexpr int KB_ROWS = 32;
constexpr int KB_GROUPS = 64 / KB_ROWS;
constexpr int KB_WAVES = 16;
constexpr int KB_CHUNK = 16;
static_assert(KB_GROUPS == 2, "the group sums meet in one exchange");

template <bool MISS>
__global__ __launch_bounds__(KB_WAVES * 64) void decode_combine_kernel(
    const float* __restrict__ x, const int32_t* __restrict__ slot, const float* __restrict__ w,
    int T, int k, int d, int nslices, int has_shared, const float* __restrict__ part,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ host_slot, int n_experts,
    int max_rank, int n_slots, float* __restrict__ y) {
  extern __shared__ float red[];  // [k+1][KB_ROWS]
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rr = lane % KB_ROWS, g = lane / KB_ROWS;
  const int r = blockIdx.x * KB_ROWS + rr;
  const int ti = min(lane, k - 1);
  int sp = slot[t * k + ti];                     // lane i < k: slot of term i
  float wv = w[t * k + ti];                      // lane i < k: weight of term i
  if (MISS) {
    const int hs = host_slot[min(max(idx[t * k + ti], 0), n_experts - 1)];
    sp = sp < 0 && ti < max_rank && hs < n_slots ? hs : -1;
  }
  const float xr = MISS ? y[static_cast<int64_t>(t) * d + r] : x[static_cast<int64_t>(t) * d + r];
  // sp and wv are read across lanes inside branches only some lanes take:
  // pinned here, with every lane active, so their definitions stay outside
  opaque(sp);
  opaque(wv);
  const int per = (nslices + KB_GROUPS - 1) / KB_GROUPS;
  const int j0 = min(nslices, g * per), j1 = min(nslices, j0 + per);
  for (int i = wave; i < k + 1; i += KB_WAVES) {
    if (MISS && (i < k ? __builtin_amdgcn_readlane(sp, i) < 0 : !has_shared)) continue;
    const float* src = part + ((static_cast<int64_t>(t) * (k + 1) + i) * nslices) * d + r;
    float acc = 0.0f;
    for (int j = j0; j < j1; j += KB_CHUNK) {
      float v[KB_CHUNK];
#pragma unroll
      for (int q = 0; q < KB_CHUNK; ++q)
        v[q] = src[static_cast<int64_t>(min(j + q, j1 - 1)) * d];
#pragma unroll
      for (int q = 0; q < KB_CHUNK; ++q) acc += j + q < j1 ? v[q] : 0.0f;
    }
    acc += __shfl_xor(acc, KB_ROWS, 64);        // g0 + g1
    if (g == 0) red[i * KB_ROWS + rr] = acc;
  }
  __syncthreads();
  if (wave != 0 || g != 0) return;
  float acc = xr;
  for (int i = 0; i < k; ++i)
    if (__builtin_amdgcn_readlane(sp, i) >= 0)
      acc = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wv), i)),
                 red[i * KB_ROWS + rr], acc);
  if (has_shared) acc += red[k * KB_ROWS + rr];
  y[static_cast<int64_t>(t) * d + r] = acc;
}

size_t part_bytes(int d, int f, int T, int k) {
  return static_cast<size_t>(static_cast<int64_t>(T) * (k + 1) * (f / SLICE) * d * 4);
}

template <int FMT, int MODE>
hipError_t launch_ffn(const FfnArgs& a, const float* x, hipStream_t s) {
  // members (T*k pairs, the shared expert), plus the side row in kAcc mode
  const dim3 grid(a.f / SLICE, a.T * a.k + (MODE == kMiss ? 0 : MODE == kAcc ? 2 : 1));
  const int upw = (a.d / 64 + KA_WAVES - 1) / KA_WAVES;
  if (upw <= 1)
    decode_ffn_kernel<FMT, 1, MODE><<<grid, KA_THREADS, 0, s>>>(a, x);
  else
    decode_ffn_kernel<FMT, 2, MODE><<<grid, KA_THREADS, 0, s>>>(a, x);
  return hipGetLastError();
}

FfnArgs ffn_args(const moe_layer& L, int T, const int32_t* slot, void* ws) {
  const SlotLayout lay = slot_layout(L.fmt, L.d_model, L.d_ff);
  FfnArgs a = {};
  a.pool = static_cast<const uint8_t*>(L.pool);
  a.slot_bytes = L.slot_bytes;
  a.G = lay.G;
  a.D = lay.D;
  a.d = L.d_model;
  a.f = L.d_ff;
  a.T = T;
  a.k = L.top_k;
  a.shared_slot = L.shared_slot;
  a.slot = slot;
  a.part = static_cast<float*>(ws);
  a.E = L.n_experts;
  return a;
}

template <int MODE>
hipError_t launch_ffn_fmt(int fmt, const FfnArgs& a, const float* x, hipStream_t s) {
  switch (fmt) {
    case MOE_FMT_Q2S: return launch_ffn<MOE_FMT_Q2S, MODE>(a, x, s);
    case MOE_FMT_Q2SM: return launch_ffn<MOE_FMT_Q2SM, MODE>(a, x, s);
    case MOE_FMT_Q3G: return launch_ffn<MOE_FMT_Q3G, MODE>(a, x, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine_partials(const moe_layer& L, const float* x, int T,
                                   const int32_t* slot, const float* w, const float* part,
                                   float* y, hipStream_t s) {
  const dim3 grid(L.d_model / KB_ROWS, T);
  const size_t lds = static_cast<size_t>(L.top_k + 1) * KB_ROWS * 4;
  decode_combine_kernel<false><<<grid, KB_WAVES * 64, lds, s>>>(
      x, slot, w, T, L.top_k, L.d_model, L.d_ff / SLICE, L.shared_slot >= 0 ? 1 : 0, part,
      nullptr, nullptr, 1, 0, 0, y);
  return hipGetLastError();
}

hipError_t launch_combine_misses(const moe_layer& H, int T, const int32_t* idx,
                                 const int32_t* slot, const float* w, const int32_t* host_slot,
                                 int max_rank, const float* part, float* y, hipStream_t s) {
  const dim3 grid(H.d_model / KB_ROWS, T);
  const size_t lds = static_cast<size_t>(H.top_k + 1) * KB_ROWS * 4;
  decode_combine_kernel<true><<<grid, KB_WAVES * 64, lds, s>>>(
      nullptr, slot, w, T, H.top_k, H.d_model, H.d_ff / SLICE, 0, part, idx, host_slot,
      H.n_experts, max_rank, H.n_slots, y);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(int d, int f, int T, int k) {
  return static_cast<size_t>(align256(static_cast<int64_t>(part_bytes(d, f, T, k))));
}

hipError_t launch_decode(const moe_layer& L, const float* x, int T, const int32_t* idx,
                         const int32_t* slot, const float* w, float* y, void* ws,
                         hipStream_t s) {
  (void)idx;
  const FfnArgs a = ffn_args(L, T, slot, ws);
  const hipError_t e = launch_ffn_fmt<kPairs>(L.fmt, a, x, s);
  if (e != hipSuccess) return e;
  return launch_combine_partials(L, x, T, slot, w, a.part, y, s);
}

hipError_t launch_decode_layer(const moe_layer& L, const float* x, int T, const float* logits,
                               const int32_t* slot_of_expert, int32_t* idx, float* w,
                               int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                               int32_t* n_miss, float* y, void* ws, hipStream_t s) {
  FfnArgs a = ffn_args(L, T, nullptr, ws);
  a.logits = logits;
  a.table = slot_of_expert;
  a.o_idx = idx;
  a.o_w = w;
  a.o_slot = slot;
  a.o_miss_expert = miss_expert;
  a.o_miss_pair = miss_pair;
  a.o_n_miss = n_miss;
  const hipError_t e = launch_ffn_fmt<kRoute>(L.fmt, a, x, s);
  if (e != hipSuccess) return e;
  return launch_combine_partials(L, x, T, slot, w, a.part, y, s);
}

hipError_t launch_decode_layer_acc(const moe_layer& L, const float* x, int T, const float* logits,
                                   const int32_t* slot_of_expert, int32_t* idx, float* w,
                                   int32_t* slot, int32_t* miss_expert, int32_t* miss_pair,
                                   int32_t* n_miss, float* acc_out, float* acc_clear,
                                   const float* prev_x, const float* prev_acc, float* prev_y,
                                   hipStream_t s) {
  FfnArgs a = ffn_args(L, T, nullptr, nullptr);
  a.logits = logits;
  a.table = slot_of_expert;
  a.o_idx = idx;
  a.o_w = w;
  a.o_slot = slot;
  a.o_miss_expert = miss_expert;
  a.o_miss_pair = miss_pair;
  a.o_n_miss = n_miss;
  a.acc_out = acc_out;
  a.acc_clear = acc_clear;
  a.prev_x = prev_x;
  a.prev_acc = prev_acc;
  a.prev_y = prev_y;
  return launch_ffn_fmt<kAcc>(L.fmt, a, x, s);
}

hipError_t launch_acc_finish(const float* x, const float* acc, int T, int d, float* y,
                             hipStream_t s) {
  acc_finish_kernel<<<T, KA_THREADS, 0, s>>>(x, acc, T, d, y);
  return hipGetLastError();
}

hipError_t launch_decode_misses(const moe_layer& H, const void* host_pool_dev, const float* x,
                                int T, const int32_t* idx, const int32_t* slot, const float* w,
                                const int32_t* host_slot_of_expert, int max_rank, float* y,
                                void* ws, hipStream_t s) {
  FfnArgs a = ffn_args(H, T, slot, ws);
  a.pool = static_cast<const uint8_t*>(host_pool_dev);
  a.shared_slot = -1;
  a.table = host_slot_of_expert;
  a.idx = idx;
  a.max_rank = max_rank;
  a.n_slots = H.n_slots;
  const hipError_t e = launch_ffn_fmt<kMiss>(H.fmt, a, x, s);
  if (e != hipSuccess) return e;
  return launch_combine_misses(H, T, idx, slot, w, host_slot_of_expert, max_rank, a.part, y, s);
}

}  // namespace bitffn
