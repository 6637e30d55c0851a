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
//    activation x is the same for all lanes (read from LDS, one address per
//    wavefront).  The 16 wavefronts split the d_model columns in interleaved
//    64-column units; their row sums meet in LDS in a fixed order, and
//    h = silu(g) * u is formed for the 32 h indices.
//    Down, split over d_ff: the same workgroup multiplies its 32 h values into
//    block column js of D (all d_model rows) and stores that partial product,
//    written through the L2 to memory.
//    Weight bytes of both parts are loaded before any arithmetic.  When there
//    are more jobs than two per CU (T >= 3 at top-10), each routing workgroup
//    takes its pair jobs in turn after routing once.
// 2. combine kernel: y[t] = x[t] + sum_i w[t,i] * (sum over slices of the
//    partials of member u(t,i)) + (same for the shared member), slices summed
//    in a fixed tree, terms in k-slot order, shared last.
// Arithmetic per block: codes become fp16 pairs (c + q) by mask-and-OR with
// an exponent, each multiplied into fp32 by v_fma_mix; the block's offset sum
// and scale/min are applied once per block.
//
// Modes of the ffn kernel: the pair slots given (moe_expert_ffn_decode), the
// routing done inside every workgroup (moe_decode_layer, moe_decode_stack),
// the missed pairs only, with their slots in a second pool such as pinned host
// memory (moe_decode_misses, whose combine adds into y), or routing with both
// pools at once (moe_decode_layer_tiers): a chosen expert missing from the
// first pool is a union member read from the second, its slot h carried as
// -2 - h, so the two kinds of member never share a slot value and the layer
// costs the slower of the two reads, not their sum.
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
  kRouteTiers = 3,   // routing in the kernel; hits from the pool, misses from the host tier
};

// Plane offsets within a slot (a slot is far below 4 GiB), 32-bit so that a
// load address is the slot base (scalar) plus a 32-bit offset.
struct Planes32 {
  uint32_t codes, hi, scale, min;
};

struct FfnArgs {
  const uint8_t* pool;
  int64_t slot_bytes;
  Planes32 G, D;
  int d, f, T, k, shared_slot;
  const int32_t* slot;
  float* part;  // [T][k+1][f/32][d]: term i of token t, the shared expert at i = k
  uint32_t part_bytes;
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
  // slot of each expert, and a miss of k-slot i runs only if i < max_rank
  const int32_t* idx;           // [T][k]
  int max_rank;
  // slots of the pool read here (the host tier's in the miss mode): a slot
  // outside [0, n_slots), whether given or looked up, counts as a miss
  int n_slots;
  // two-tier routing mode only: the host tier (same layout and slot size),
  // the host slot of each expert, and the tier's slot count
  const uint8_t* host_pool;
  const int32_t* host_table;    // [E]
  int host_n_slots;
};

// Routing inside the kernel: experts are taken in chunks of 512, one
// wavefront per (token, chunk) holding 8 keys per lane; each chunk's top k is
// found by wave_topk_keys, and with two chunks a second pass ranks the 2k
// survivors of each token.
constexpr int kRouteChunk = 512;
constexpr int kRouteChunks = (MOE_MAX_EXPERTS + kRouteChunk - 1) / kRouteChunk;
static_assert(MOE_MAX_EXPERTS <= KA_THREADS, "one slot-table entry per thread");
static_assert(MOE_MAX_DECODE_T * kRouteChunks <= KA_WAVES, "one wavefront per token and chunk");
static_assert(kRouteChunks <= 2, "at most two chunks (the merge holds 2 keys per lane)");

// Jobs of the shared expert per slice: one (it serves every token), none
// without a shared expert or in the miss mode.
__host__ __device__ inline int shared_jobs_per_slice(int shared_slot, bool miss) {
  return (miss || shared_slot < 0) ? 0 : 1;
}

// Union member u: its slot, the mask of tokens it serves, and `same`, the
// mask of pairs naming that slot (all of them for the shared expert, whose
// term is i = k).  `sp` is the slot of pair `lane` (-1 for lanes >= T*k;
// T*k <= 64), so the test is a lane read and a ballot; the result is uniform
// across the wavefront.
__device__ __forceinline__ bool union_member(int sp, int T, int k, int shared_slot, int u,
                                             int& s, uint32_t& mask, uint64_t& same,
                                             bool host_members = false) {
  const int n = T * k;
  if (u == n) {
    if (shared_slot < 0) return false;
    s = shared_slot;
    mask = (1u << T) - 1u;
    same = 0;
    return true;
  }
  s = __builtin_amdgcn_readlane(sp, u);
  if (host_members ? s == -1 : s < 0) return false;
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
// member.
template <int FMT, int UPW, int MODE, bool LOOP>
__global__ __launch_bounds__(KA_THREADS) __attribute__((amdgpu_num_sgpr(72), amdgpu_waves_per_eu(8, 8))) void decode_ffn_kernel(FfnArgs a,
                                                                const float* __restrict__ x) {
  constexpr bool ROUTE = MODE == kRoute || MODE == kRouteTiers;
  constexpr bool TIERS = MODE == kRouteTiers;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar addressing
  const int d = a.d;
  const int n = a.T * a.k;
  int sp = -1;   // slot of pair `lane`
  if (MODE == kPairs) {
    const int gs = a.slot[min(lane, n - 1)];
    sp = lane < n && gs < a.n_slots ? gs : -1;
  }
  if (MODE == kMiss) {
    const int p = min(lane, n - 1);
    const int gpu_slot = a.slot[p];
    const int e = min(max(a.idx[p], 0), a.E - 1);
    const int hs = a.table[e];
    sp = lane < n && gpu_slot < 0 && p % a.k < a.max_rank && hs < a.n_slots ? hs : -1;
  }

  // Every load below is unconditional, with indices clamped into range (the
  // surplus values are never used), so the compiler can count outstanding
  // loads and wait for each group alone.  First x and the routing inputs.
  float2 xv[MOE_MAX_DECODE_T];
  const int ex = min(2 * tid, d - 2);
#pragma unroll
  for (int t = 0; t < MOE_MAX_DECODE_T; ++t)   // uniform: only the T tokens' rows
    xv[t] = t < a.T ? *reinterpret_cast<const float2*>(x + static_cast<int64_t>(t) * d + ex)
                    : make_float2(0.0f, 0.0f);
  const int nslices = a.f / SLICE;
  // Jobs: first the shared expert's, one per slice js at j = js, then one
  // per (pair u, slice js) at j = n_shared + u * nslices + js.  A workgroup
  // of a shared job does only that job (it serves every token, the longest
  // job) and skips routing; the others take the pair jobs in turn.
  const int n_shared = shared_jobs_per_slice(a.shared_slot, MODE == kMiss) * nslices;
  const int n_jobs = n_shared + n * nslices;
  const bool routing = ROUTE && static_cast<int>(blockIdx.x) >= n_shared;   // uniform
  const int nchunk = (a.E + kRouteChunk - 1) / kRouteChunk;
  const int rt = wave / kRouteChunks, rc = wave % kRouteChunks;   // token and chunk of a routing wave
  const bool route_wave = routing && rt < a.T && rc < nchunk;
  float lg[8] = {};
  int tv = 0;
  if (ROUTE) {
    const int tt = min(rt, a.T - 1);
    if (route_wave)   // uniform: the logits only in the wavefronts that rank them
#pragma unroll
    for (int j = 0; j < 8; ++j)
      lg[j] = a.logits[static_cast<int64_t>(tt) * a.E + min(rc * kRouteChunk + 64 * j + lane, a.E - 1)];
    tv = a.table[min(tid, a.E - 1)];
    if (TIERS) {   // an expert missing from the pool: its host slot, encoded as -2 - h
      const int hs = a.host_table[min(tid, a.E - 1)];
      tv = (tv >= 0 && tv < a.n_slots) ? tv : (hs >= 0 && hs < a.host_n_slots ? -2 - hs : -1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // keep the issue order

  __shared__ __attribute__((aligned(16))) float s_x[MOE_MAX_DECODE_T][2048];
  __shared__ float2 bsum[MOE_MAX_DECODE_T][2048 / 32];   // per block of x: (sum, offset constant)
  __shared__ uint64_t s_cand[MOE_MAX_DECODE_T * kRouteChunks * MOE_MAX_TOPK];
  __shared__ uint64_t s_top[MOE_MAX_DECODE_PAIRS];
  __shared__ uint64_t s_scr[MOE_MAX_DECODE_T * kRouteChunks][128];
  __shared__ int32_t s_table[MOE_MAX_EXPERTS];

  // x into LDS (the gate/up products read it from there), and per-block sums
  // of x (sum, offset constant) for every token: each thread adds two
  // neighbouring values, the 16 threads of a block reduce by DPP rotations
  // within their row of 16 lanes; lane 0 of the row stores
  const float cw0 = block_offset_weight<FMT>(ex & 31), cw1 = block_offset_weight<FMT>((ex & 31) + 1);
#pragma unroll
  for (int t = 0; t < MOE_MAX_DECODE_T; ++t) {
    if (t < a.T && 2 * tid < d) *reinterpret_cast<float2*>(&s_x[t][2 * tid]) = xv[t];
    const float sx = row16_sum(xv[t].x + xv[t].y);
    const float sc = row16_sum(fmaf(cw1, xv[t].y, cw0 * xv[t].x));
    if (t < a.T && (tid & 15) == 0 && 2 * tid < d)
      bsum[t][tid >> 4] = make_float2(sx, block_const<FMT>(sx, sc));
  }

  if (ROUTE) {
    if (route_wave) {   // top k of chunk rc of token rt
      uint64_t key[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = rc * kRouteChunk + 64 * j + lane;
        key[j] = route_key(lg[j], e, e < a.E);
      }
      uint64_t* out = nchunk == 1 ? s_top + rt * a.k : s_cand + (rt * kRouteChunks + rc) * a.k;
      wave_topk_keys<8>(key, a.k, out, s_scr[wave]);
    }
    if (tid < a.E) s_table[tid] = tv < a.n_slots ? tv : -1;   // out of the pool: a miss
                                                            // (or its encoded host slot)
  }
  __syncthreads();
  if (ROUTE && nchunk > 1) {   // uniform: rank the 2k survivors of each token
    if (routing && wave < a.T) {
      uint64_t key[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        key[h] = lane < a.k ? s_cand[(wave * kRouteChunks + h) * a.k + lane] : 0ull;
      wave_topk_keys<2>(key, a.k, s_top + wave * a.k, s_scr[wave]);
    }
    __syncthreads();
  }
  if (routing) {
    const int e = lane < n ? key_expert(s_top[lane]) : 0;
    sp = lane < n ? s_table[e] : -1;
    const int gpu_sp = sp < 0 ? -1 : sp;   // the pool's slot (-1: a miss)
    if (TIERS && sp < -1 && lane % a.k >= a.max_rank) sp = -1;   // a miss left out
    if (static_cast<int>(blockIdx.x) == n_shared) {   // routing outputs: the first routing workgroup
      if (wave < a.T) {
        int id;
        float wt;
        topk_softmax_lane(s_top + wave * a.k, a.k, lane, id, wt);
        if (lane < a.k) {
          a.o_idx[wave * a.k + lane] = id;
          a.o_w[wave * a.k + lane] = wt;
          a.o_slot[wave * a.k + lane] = max(s_table[id], -1);
        }
      }
      if (wave == KA_WAVES - 1)
        wave_miss_lists(lane, n, e, gpu_sp, a.o_miss_expert, a.o_miss_pair, a.o_n_miss);
    }
  }

  __shared__ float red[KA_WAVES][64];
  __shared__ __attribute__((aligned(16))) float hsh[SLICE];
  __shared__ float hsum[2];
  // the pair slots, kept in LDS for the jobs: every wavefront holds the same
  // values and writes them to the same place, then reads back its own lane,
  // so no barrier is needed, and no register holds them across a job loop
  __shared__ int32_t s_sp[64];
  s_sp[lane] = sp;

  // one job; LOOP: the workgroup takes jobs blockIdx.x, + gridDim.x, ...,
  // else exactly one (grid = jobs), with no loop around the job's code
  auto run_job = [&](int job) {
  const bool shared_job = job < n_shared;
  const int u = shared_job ? n : (job - n_shared) / nslices;
  const int js = shared_job ? job : (job - n_shared) % nslices;
  // the thread index, opaque here so that the per-thread offsets below are
  // formed in each job instead of being kept (and spilled) across jobs
  int tj = tid;
  opaque(tj);
  int s;
  uint32_t mask;
  uint64_t same;
  if (!union_member(s_sp[tj & 63], a.T, a.k, a.shared_slot, u, s, mask, same, TIERS)) return;
  const uint8_t* __restrict__ base =
      TIERS && s < 0 ? a.host_pool + static_cast<int64_t>(-2 - s) * a.slot_bytes
                     : a.pool + static_cast<int64_t>(s) * a.slot_bytes;
  const uint32_t R = 2u * static_cast<uint32_t>(a.f);                   // G rows
  const uint32_t grow = 2u * SLICE * js + static_cast<uint32_t>(tj & 63);   // this lane's G row
  const int nu = d / 64;

  // ---- loads: G units of this wavefront, then D block column js ----
  uint4 gc[UPW];
  uint32_t gs[UPW], gm[UPW];
  uint2 gh[UPW];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const uint32_t unit = static_cast<uint32_t>(min(wave + KA_WAVES * i, nu - 1)) * R + grow;
    gc[i] = stream_u4(base + (a.G.codes + unit * 16u));
    gs[i] = stream_u32(base + (a.G.scale + unit * 4u));
    if (FMT == MOE_FMT_Q2SM) gm[i] = stream_u32(base + (a.G.min + unit * 4u));
    if (FMT == MOE_FMT_Q3G) gh[i] = stream_u2(base + (a.G.hi + unit * 8u));
  }
  __builtin_amdgcn_sched_barrier(0);
  const int ndr = (d - tj + KA_THREADS - 1) / KA_THREADS;   // D rows of this thread
  uint2 dc[MAX_DROWS];
  uint32_t ds[MAX_DROWS], dm[MAX_DROWS], dh[MAX_DROWS];
#pragma unroll
  for (int i = 0; i < MAX_DROWS; ++i) {
    const uint32_t unit = static_cast<uint32_t>(js * d + min(tj + KA_THREADS * i, d - 1));
    dc[i] = stream_u2(base + (a.D.codes + unit * 8u));
    ds[i] = stream_u16(base + (a.D.scale + unit * 2u));
    if (FMT == MOE_FMT_Q2SM) dm[i] = stream_u16(base + (a.D.min + unit * 2u));
    if (FMT == MOE_FMT_Q3G) dh[i] = stream_u32(base + (a.D.hi + unit * 4u));
  }

  // one served token: gate/up, SiLU gating, partial down product
  auto token_pass = [&](int t) {
    // gate/up rows: partial sums over this wavefront's units (x read from
    // LDS, the same address in every lane)
    float row = 0.0f;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int c = wave + KA_WAVES * i;
      if (c < nu) {
        const float* xw = &s_x[t][64 * c];
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
    // this row of partials, addressed through a buffer resource over the
    // partials (32-bit offsets, so the stores need one VGPR each)
    const uint32_t obase = static_cast<uint32_t>(((t * (a.k + 1) + term) * nslices + js) * d) * 4u;
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(a.part, 0, static_cast<int>(a.part_bytes), 0x00020000);
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
        // written through to memory (cache policy SC1, device scope: bit 4
        // of the policy operand on gfx950): the combine reads the partials
        // on other XCDs, and lines left dirty in this XCD's L2 would have to
        // be written back when the kernel ends, before the combine starts
        __builtin_amdgcn_raw_buffer_store_b32(
            __builtin_bit_cast(uint32_t, v), prs,
            static_cast<int>(obase + 4u * static_cast<uint32_t>(tid + KA_THREADS * i)), 0, 16);
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
  };   // run_job
  if (LOOP && static_cast<int>(blockIdx.x) >= n_shared) {
    const int stride = static_cast<int>(gridDim.x) - n_shared;
    for (int job = blockIdx.x; job < n_jobs; job += stride) run_job(job);
  } else if (static_cast<int>(blockIdx.x) < n_jobs) {
    run_job(blockIdx.x);
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

// CM: kCombinePlain (y = x + terms), kCombineMisses (y += the host tier's
// terms), kCombineTiers (y = x + the pool's and the host tier's terms).
enum CombineMode { kCombinePlain = 0, kCombineMisses = 1, kCombineTiers = 2 };
template <int CM>
__global__ __launch_bounds__(KB_WAVES * 64) void decode_combine_kernel(
    const float* __restrict__ x, const int32_t* __restrict__ slot, const float* __restrict__ w,
    int T, int k, int d, int nslices, int has_shared, const float* __restrict__ part,
    const int32_t* __restrict__ idx, const int32_t* __restrict__ host_slot, int n_experts,
    int max_rank, int n_slots, float* __restrict__ y, float* __restrict__ xnext,
    const float* __restrict__ addend) {
  extern __shared__ float red[];  // [k+1][KB_ROWS]
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rr = lane % KB_ROWS, g = lane / KB_ROWS;
  const int r = blockIdx.x * KB_ROWS + rr;
  const int ti = min(lane, k - 1);
  int sp = slot[t * k + ti];                     // lane i < k: slot of term i
  float wv = w[t * k + ti];                      // lane i < k: weight of term i
  constexpr bool MISS = CM == kCombineMisses;
  if (CM != kCombinePlain) {   // n_slots: the host tier's
    const int hs = host_slot[min(max(idx[t * k + ti], 0), n_experts - 1)];
    const int hm = ti < max_rank && hs >= 0 && hs < n_slots ? hs : -1;   // a miss that ran
    // the two-tier layer's slot output is the pool's slot (-1: a miss), in range
    sp = MISS ? (sp < 0 ? hm : -1) : (sp >= 0 ? sp : hm);
  } else {
    sp = sp < n_slots ? sp : -1;   // a slot outside the pool is a miss, as in the ffn kernel
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
  const int64_t o = static_cast<int64_t>(t) * d + r;
  if (y) y[o] = acc;
  // the next layer's input, when the step continues: y + addend
  if (xnext) xnext[o] = addend ? acc + addend[o] : acc;
}

size_t part_bytes(int d, int f, int T, int k) {
  return static_cast<size_t>(static_cast<int64_t>(T) * (k + 1) * (f / SLICE) * d * 4);
}

// Workgroups of the ffn kernel: one per job if all fit at two workgroups per
// CU (two fit together), else one per shared job plus the fewest rounds of
// the pair jobs over the other places, spread evenly.
struct FfnGrid {
  int jobs, grid;
};
FfnGrid ffn_grid(int T, int k, int f, int shared_slot, bool miss) {
  const int nslices = f / SLICE;
  const int n_shared = shared_jobs_per_slice(shared_slot, miss) * nslices;
  const int n_pair = T * k * nslices;
  const int slots = 2 * device_cus();
  if (n_shared + n_pair <= slots || slots <= n_shared) return {n_shared + n_pair, n_shared + n_pair};
  const int rounds = (n_pair + (slots - n_shared) - 1) / (slots - n_shared);
  return {n_shared + n_pair, n_shared + (n_pair + rounds - 1) / rounds};
}

template <int FMT, int MODE>
hipError_t launch_ffn(const FfnArgs& a, const float* x, hipStream_t s) {
  const FfnGrid g = ffn_grid(a.T, a.k, a.f, a.shared_slot, MODE == kMiss);
  const int jobs = g.jobs, grid = g.grid;
  const int upw = (a.d / 64 + KA_WAVES - 1) / KA_WAVES;
  // the job loop only where a workgroup takes more than one job (routing
  // mode: one routing per workgroup for all its jobs)
  if constexpr (MODE == kRoute || MODE == kRouteTiers) {
    if (grid < jobs) {
      if (upw <= 1)
        decode_ffn_kernel<FMT, 1, MODE, true><<<grid, KA_THREADS, 0, s>>>(a, x);
      else
        decode_ffn_kernel<FMT, 2, MODE, true><<<grid, KA_THREADS, 0, s>>>(a, x);
      return hipGetLastError();
    }
  }
  {
    if (upw <= 1)
      decode_ffn_kernel<FMT, 1, MODE, false><<<jobs, KA_THREADS, 0, s>>>(a, x);
    else
      decode_ffn_kernel<FMT, 2, MODE, false><<<jobs, KA_THREADS, 0, s>>>(a, x);
  }
  return hipGetLastError();
}

FfnArgs ffn_args(const moe_layer& L, int T, const int32_t* slot, void* ws) {
  const SlotLayout lay = slot_layout(L.fmt, L.d_model, L.d_ff);
  FfnArgs a = {};
  a.pool = static_cast<const uint8_t*>(L.pool);
  a.slot_bytes = L.slot_bytes;
  auto p32 = [](const Planes& P) {
    return Planes32{static_cast<uint32_t>(P.codes), static_cast<uint32_t>(P.hi),
                    static_cast<uint32_t>(P.scale), static_cast<uint32_t>(P.min)};
  };
  a.G = p32(lay.G);
  a.D = p32(lay.D);
  a.d = L.d_model;
  a.f = L.d_ff;
  a.T = T;
  a.k = L.top_k;
  a.shared_slot = L.shared_slot;
  a.slot = slot;
  a.part = static_cast<float*>(ws);
  a.part_bytes = static_cast<uint32_t>(part_bytes(L.d_model, L.d_ff, T, L.top_k));
  a.E = L.n_experts;
  a.n_slots = L.n_slots;
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
                                   float* y, hipStream_t s, float* xnext = nullptr,
                                   const float* addend = nullptr) {
  const dim3 grid(L.d_model / KB_ROWS, T);
  const size_t lds = static_cast<size_t>(L.top_k + 1) * KB_ROWS * 4;
  decode_combine_kernel<kCombinePlain><<<grid, KB_WAVES * 64, lds, s>>>(
      x, slot, w, T, L.top_k, L.d_model, L.d_ff / SLICE, L.shared_slot >= 0 ? 1 : 0, part,
      nullptr, nullptr, 1, 0, L.n_slots, y, xnext, addend);
  return hipGetLastError();
}

hipError_t launch_combine_tiers(const moe_layer& L, const moe_layer& H, const float* x, int T,
                               const int32_t* idx, const int32_t* slot, const float* w,
                               const int32_t* host_slot, int max_rank, const float* part,
                               float* y, hipStream_t s) {
  const dim3 grid(L.d_model / KB_ROWS, T);
  const size_t lds = static_cast<size_t>(L.top_k + 1) * KB_ROWS * 4;
  decode_combine_kernel<kCombineTiers><<<grid, KB_WAVES * 64, lds, s>>>(
      x, slot, w, T, L.top_k, L.d_model, L.d_ff / SLICE, L.shared_slot >= 0 ? 1 : 0, part, idx,
      host_slot, L.n_experts, max_rank, H.n_slots, y, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_combine_misses(const moe_layer& H, int T, const int32_t* idx,
                                 const int32_t* slot, const float* w, const int32_t* host_slot,
                                 int max_rank, const float* part, float* y, hipStream_t s) {
  const dim3 grid(H.d_model / KB_ROWS, T);
  const size_t lds = static_cast<size_t>(H.top_k + 1) * KB_ROWS * 4;
  decode_combine_kernel<kCombineMisses><<<grid, KB_WAVES * 64, lds, s>>>(
      nullptr, slot, w, T, H.top_k, H.d_model, H.d_ff / SLICE, 0, part, idx, host_slot,
      H.n_experts, max_rank, H.n_slots, y, nullptr, nullptr);
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
                               int32_t* n_miss, float* y, void* ws, hipStream_t s, float* xnext,
                               const float* addend) {
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
  return launch_combine_partials(L, x, T, slot, w, a.part, y, s, xnext, addend);
}

hipError_t launch_decode_layer_tiers(const moe_layer& L, const moe_layer& H,
                                     const void* host_pool_dev, const int32_t* host_slot_of_expert,
                                     int max_rank, const float* x, int T, const float* logits,
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
  a.max_rank = max_rank;
  a.host_pool = static_cast<const uint8_t*>(host_pool_dev);
  a.host_table = host_slot_of_expert;
  a.host_n_slots = H.n_slots;
  const hipError_t e = launch_ffn_fmt<kRouteTiers>(L.fmt, a, x, s);
  if (e != hipSuccess) return e;
  return launch_combine_tiers(L, H, x, T, idx, slot, w, host_slot_of_expert, max_rank, a.part,
                              y, s);
}

hipError_t launch_decode_misses(const moe_layer& H, const void* host_pool_dev, const float* x,
                                int T, const int32_t* idx, const int32_t* slot, const float* w,
                                const int32_t* host_slot_of_expert, int max_rank, float* y,
                                void* ws, hipStream_t s, int phases) {
  FfnArgs a = ffn_args(H, T, slot, ws);
  a.pool = static_cast<const uint8_t*>(host_pool_dev);
  a.shared_slot = -1;
  a.table = host_slot_of_expert;
  a.idx = idx;
  a.max_rank = max_rank;
  a.n_slots = H.n_slots;
  if (phases & MOE_MISSES_READ) {
    const hipError_t e = launch_ffn_fmt<kMiss>(H.fmt, a, x, s);
    if (e != hipSuccess) return e;
  }
  if (phases & MOE_MISSES_JOIN)
    return launch_combine_misses(H, T, idx, slot, w, host_slot_of_expert, max_rank, a.part, y, s);
  return hipSuccess;
}

}  // namespace bitffn
