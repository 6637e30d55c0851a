// Decode / verify through a stack of MoE layers in one persistent kernel.
//
// The grid is one workgroup of 16 wavefronts per compute unit, all resident
// at once (cooperative launch).  Per layer l every workgroup
//   1. has the layer's routing (top-k of the logits, slot lookup, the union
//      of the chosen resident experts plus the shared one: the members);
//   2. gate/up phase: computes h = silu(G_gate x) * (G_up x) for its share of
//      the (member, h index) space and stores it (sc1 stores, visible at
//      agent scope);
//   3. barrier H (all h of the layer stored);
//   4. down phase: for one token and a range of output rows, the down
//      product of every term of that token (its k chosen resident experts in
//      k-slot order, then the shared one), each over the d_ff blocks in
//      order, then y = x + sum_i w_i o_i + o_shared; stores y and the next
//      layer's input x' = y + addend';
//   5. barrier Y (all of x' stored) before the next layer's gate/up phase.
// Routing of layer l+1 uses only that layer's logits and slot table, so by
// default every workgroup computes it while it waits at barrier H of layer
// l; with the route-after-x flag it runs after barrier Y instead.
//
// Work split of the gate/up phase.  A tile is 32 h indices of one member
// (64 G rows); lane l of every wavefront streams row 64js + l, the 16
// wavefronts split the d_model columns in interleaved 64-column units, and
// x arrives as scalar operands (read through the constant address space).
// Tiles go round robin over the workgroups.  When only a few tiles are left
// over after whole rounds (11 members x 24 tiles = 264 on 256 CUs), those
// are split one h index per workgroup and computed with one lane per block
// (the remainder path), with the same operations in the same order as the
// tile path, so an h value has the same bits whichever path computes it.
//
// Every sum has a fixed order that depends neither on the workgroup that
// computes it nor on the other tokens of the step, so reruns are bitwise
// equal and a token verified with 3 drafts gets the bits it gets alone.
//
// Data exchange: h and x' go through buffers that are written once per
// layer at addresses no workgroup has read before in the launch (fresh per
// layer), with sc1 stores, and are read after the barrier; the barrier is a
// two-level arrival count (8 groups, then a top count) whose last arriver
// publishes the epoch.  Waits are bounded: a wait that gives up sets the
// workspace's error word, and every later wait returns at once.
#include "moe_internal.h"
#include "route_device.h"

#pragma clang fp contract(off)

namespace bitffn {
namespace {

typedef uint32_t nu4 __attribute__((ext_vector_type(4)));
typedef uint32_t nu2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) float cfloat;

__device__ __forceinline__ uint4 nt_u4(const uint8_t* p) {
  const nu4 v = __builtin_nontemporal_load(reinterpret_cast<const nu4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 nt_u2(const uint8_t* p) {
  const nu2 v = __builtin_nontemporal_load(reinterpret_cast<const nu2*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t nt_u32(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t nt_u16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __builtin_bit_cast(uint32_t, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int TILE_H = 32;                          // h indices per tile
constexpr int MAXM = MOE_MAX_DECODE_PAIRS + 1;      // members incl. the shared one
constexpr int NGROUPS = 8;                          // first level of the barrier
constexpr unsigned SPIN_CAP = 1u << 21;             // polls before a wait gives up
constexpr int RMAX = 64;                            // output rows per down pass
constexpr int B_BUDGET = 80 * 1024;                 // LDS bytes for h, block sums, parts

// sync words (uint32 index): error, generation, group counts, top count, epoch
constexpr int SY_ERR = 0, SY_GEN = 32, SY_GROUP = 64, SY_TOP = SY_GROUP + 32 * NGROUPS,
              SY_READY = SY_TOP + 32;

struct Members {
  int n_routed, n_m, pad0, pad1;
  int slot[MAXM];
  uint32_t mask[MAXM];               // tokens served
  int pm[MOE_MAX_DECODE_PAIRS];      // pair t*k+i -> member, -1 = miss
  float w[MOE_MAX_DECODE_PAIRS];     // routing weight of pair t*k+i
};

struct LdsLayout {
  // byte offsets into the dynamic LDS block
  int grp, cand, top, table, mem, bsum, red, racc, rs16, rm16, red2, tq, b, obuf, total;
};

__host__ __device__ constexpr int a16(int n) { return (n + 15) & ~15; }

__host__ __device__ constexpr LdsLayout lds_layout() {
  LdsLayout L{};
  int p = 0;
  L.grp = p;   p += a16(NW * 64 * 8);
  L.cand = p;  p += a16((MOE_MAX_EXPERTS / 64) * MOE_MAX_DECODE_PAIRS * 8);
  L.top = p;   p += a16(MOE_MAX_DECODE_PAIRS * 8);
  L.table = p; p += a16(MOE_MAX_EXPERTS * 4);
  L.mem = p;   p += a16(2 * static_cast<int>(sizeof(Members)));
  L.bsum = p;  p += a16(MOE_MAX_DECODE_T * 64 * 8);
  L.red = p;   p += a16(NW * 64 * 4);
  L.racc = p;  p += a16(2 * 64 * 4);
  L.rs16 = p;  p += a16(2 * 64 * 4);
  L.rm16 = p;  p += a16(2 * 64 * 4);
  L.red2 = p;  p += a16(2 * 16 * 4);
  L.tq = p;    p += a16(2 * MAXM * 4);
  L.b = p;     p += a16(B_BUDGET);
  L.obuf = p;  p += a16(MAXM * RMAX * 4);
  L.total = p;
  return L;
}
constexpr int STACK_LDS = lds_layout().total;
static_assert(STACK_LDS <= 160 * 1024, "LDS of the stack kernel");

struct StackLayerDev {
  const uint8_t* pool;
  int64_t slot_bytes;
  const int32_t* table;
  const float* logits;
  const float* addend;
  float* y;
  int32_t* idx;
  float* w;
  int32_t* slot;
  int32_t* miss_expert;
  int32_t* miss_pair;
  int32_t* n_miss;
  int32_t n_slots, fmt, shared_slot, pad;
};

struct StackArgs {
  int d, f, E, k, T, n_layers, route_after_x, pairs_mode, nwg;
  const float* x0;             // input of this launch's first layer [T][d]
  float* xout;                 // if set: y of the last layer + addend_next, [T][d]
  const float* addend_next;
  unsigned* sync;
  float* hbuf;                 // per layer: [MAXM'][T][f], MAXM' = T*k + 1
  int64_t h_stride;            // floats per layer
  float* xbuf;                 // per layer (l >= 1): [T][d]
  int64_t x_stride;
  const int32_t* in_idx;       // pairs mode (one layer): the given routing
  const int32_t* in_slot;
  const float* in_w;
  StackLayerDev L[MOE_MAX_STACK_LAYERS];
};

// ---------------------------------------------------------------------------
// barrier
// ---------------------------------------------------------------------------

__device__ __forceinline__ unsigned ld_agent(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread's stores done, then one arrival per workgroup; the last
// arrival of a group resets the group count and arrives at the top count; the
// last top arrival resets it and publishes `epoch`.  Resets complete before
// the epoch is published, and no workgroup arrives again before it sees it.
__device__ __forceinline__ void bar_arrive(unsigned* sync, int wg, int nwg, unsigned epoch) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x != 0) return;
  const int g = wg % NGROUPS;
  const unsigned gsize = static_cast<unsigned>((nwg - g + NGROUPS - 1) / NGROUPS);
  const unsigned ng = static_cast<unsigned>(nwg < NGROUPS ? nwg : NGROUPS);
  unsigned* gc = sync + SY_GROUP + 32 * g;
  if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u != gsize)
    return;
  __hip_atomic_store(gc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  unsigned* top = sync + SY_TOP;
  if (__hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u != ng)
    return;
  __hip_atomic_store(top, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __hip_atomic_store(sync + SY_READY, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the published epoch reaches `epoch` (wrap-safe compare).  Gives
// up after SPIN_CAP polls, or at once when another wait gave up.
__device__ __forceinline__ void bar_wait(unsigned* sync, unsigned epoch) {
  if (threadIdx.x == 0) {
    unsigned n = 0;
    while (static_cast<int>(ld_agent(sync + SY_READY) - epoch) < 0) {
      if ((++n & 63u) == 0u) {
        if (ld_agent(sync + SY_ERR) != 0u) break;
        if (n > SPIN_CAP) {
          __hip_atomic_store(sync + SY_ERR, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// routing of one layer: members, routing outputs (workgroup 0)
// ---------------------------------------------------------------------------

__device__ void stack_route(const StackArgs& a, const StackLayerDev& Ld, bool pairs,
                            uint8_t* smem, const LdsLayout& LL, Members& M) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, k = a.k, E = a.E, n = T * k;
  uint64_t* s_top = reinterpret_cast<uint64_t*>(smem + LL.top);
  int32_t* s_table = reinterpret_cast<int32_t*>(smem + LL.table);
  const bool out = !pairs && blockIdx.x == 0;
  if (!pairs) {
    float lg[4];
    topk_load<4>(Ld.logits, T, E, lg);
    const int tv = Ld.table[min(tid, E - 1)];
    topk_select<4>(lg, T, E, k,
                   TopkLds{reinterpret_cast<uint64_t*>(smem + LL.grp),
                           reinterpret_cast<uint64_t*>(smem + LL.cand), s_top},
                   [&] {
                     if (tid < E) s_table[tid] = tv;
                   });
    // routing weights of every pair (wave t: token t)
    if (wave < T) {
      int id;
      float wt;
      topk_softmax_lane(s_top + wave * k, k, lane, id, wt);
      if (lane < k) {
        M.w[wave * k + lane] = wt;
        if (out && Ld.idx) {
          Ld.idx[wave * k + lane] = id;
          Ld.w[wave * k + lane] = wt;
          Ld.slot[wave * k + lane] = s_table[id];
        }
      }
    }
  }
  if (wave == 0) {
    int sp = -1, e = 0;
    if (lane < n) {
      if (pairs) {
        sp = a.in_slot[lane];
        M.w[lane] = a.in_w[lane];
      } else {
        e = key_expert(s_top[lane]);
        sp = s_table[e];
      }
    }
    // member of pair `lane`: the first pair naming the same slot
    int firstq = lane;
    for (int q = 0; q < n; ++q) {
      const int sq = __builtin_amdgcn_readlane(sp, q);
      if (q < firstq && sq == sp) firstq = q;
    }
    const bool first = sp >= 0 && firstq == lane;
    const uint64_t firsts = __ballot(first);
    const int nr = __popcll(firsts);
    const int u = __popcll(firsts & ((1ull << firstq) - 1ull));   // member index
    if (lane < n) M.pm[lane] = sp >= 0 ? u : -1;
    if (lane < MAXM) M.mask[lane] = 0u;
    if (first) M.slot[u] = sp;
    __builtin_amdgcn_wave_barrier();
    if (sp >= 0) atomicOr(&M.mask[u], 1u << (lane / k));
    if (lane == 0) {
      M.n_routed = nr;
      const bool sh = Ld.shared_slot >= 0;
      M.n_m = nr + (sh ? 1 : 0);
      if (sh) {
        M.slot[nr] = Ld.shared_slot;
        M.mask[nr] = (1u << T) - 1u;
      }
    }
    if (out && Ld.miss_expert)
      wave_miss_lists(lane, n, e, sp, Ld.miss_expert, Ld.miss_pair, Ld.n_miss);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// gate/up phase
// ---------------------------------------------------------------------------

struct TileRegs {
  uint4 c[2];
  uint32_t s[2];
  uint2 a[2];   // Q2SM: mins in .x; Q3G: high-bit words
};

template <int FMT, int UPW>
__device__ __forceinline__ void tile_load(TileRegs& r, const uint8_t* base, const Planes& G,
                                          int64_t R, int64_t grow, int wave, int nu) {
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int64_t unit = static_cast<int64_t>(min(wave + NW * i, nu - 1)) * R + grow;
    r.c[i] = nt_u4(base + G.codes + unit * 16);
    r.s[i] = nt_u32(base + G.scale + unit * 4);
    if (FMT == MOE_FMT_Q2SM) r.a[i].x = nt_u32(base + G.min + unit * 4);
    if (FMT == MOE_FMT_Q3G) r.a[i] = nt_u2(base + G.hi + unit * 8);
  }
}

// This lane's row partial over the wavefront's units (x of one token as
// scalar operands; bs: the token's per-block (sum, offset constant)).
template <int FMT, int UPW>
__device__ __forceinline__ float tile_row(const TileRegs& r, const float* xt, const float2* bs,
                                          int wave, int nu) {
  float row = 0.0f;
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int c = wave + NW * i;
    if (c < nu) {
      const cfloat* xw = (const cfloat*)(xt + 64 * c);
      const float2 s0 = bs[2 * c], s1 = bs[2 * c + 1];
      const uint32_t m = FMT == MOE_FMT_Q2SM ? r.a[i].x : 0u;
      const float acc0 =
          block_acc<FMT>(r.c[i].x, r.c[i].y, FMT == MOE_FMT_Q3G ? r.a[i].x : 0u, xw, 0);
      row = block_finish<FMT>(row, acc0, s0.y, s0.x, r.s[i], m);
      const float acc1 =
          block_acc<FMT>(r.c[i].z, r.c[i].w, FMT == MOE_FMT_Q3G ? r.a[i].y : 0u, xw, 32);
      row = block_finish<FMT>(row, acc1, s1.y, s1.x, r.s[i] >> 16, m >> 16);
    }
  }
  return row;
}

// Per-block (sum of x, offset constant) of every token of the layer input.
template <int FMT>
__device__ __forceinline__ void block_sums(const float* x, int T, int d, float2 (*bsum)[64]) {
  const int tid = threadIdx.x;
  const int ex = min(2 * tid, d - 2);
  const float cw0 = block_offset_weight<FMT>(ex & 31), cw1 = block_offset_weight<FMT>((ex & 31) + 1);
  for (int t = 0; t < T; ++t) {
    const float2 xv = *reinterpret_cast<const float2*>(x + static_cast<int64_t>(t) * d + ex);
    const float sx = row16_sum_dpp(xv.x + xv.y);
    const float sc = row16_sum_dpp(fmaf(cw1, xv.y, cw0 * xv.x));
    if ((tid & 15) == 0 && 2 * tid < d) bsum[t][tid >> 4] = make_float2(sx, block_const<FMT>(sx, sc));
  }
}

template <int FMT, int UPW>
__device__ void gateup_phase(const StackArgs& a, const StackLayerDev& Ld, const Members& M,
                             const float* xl, float* hl, uint8_t* smem, const LdsLayout& LL) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x, nwg = a.nwg;
  const int d = a.d, f = a.f, T = a.T;
  const int NJS = f / TILE_H, nu = d / 64;
  float2(*bsum)[64] = reinterpret_cast<float2(*)[64]>(smem + LL.bsum);
  float(*red)[64] = reinterpret_cast<float(*)[64]>(smem + LL.red);
  block_sums<FMT>(xl, T, d, bsum);
  __syncthreads();

  const SlotLayout lay = slot_layout(FMT, d, f);
  const int64_t R = 2 * static_cast<int64_t>(f);
  const int n_tiles = M.n_m * NJS;
  const int full = n_tiles / nwg, left = n_tiles % nwg;
  const bool remainder = full >= 1 && left > 0 && left * TILE_H <= nwg;
  const int mine = remainder ? full : (wg < n_tiles ? (n_tiles - 1 - wg) / nwg + 1 : 0);

  for (int i = 0; i < mine; ++i) {
    const int tau = wg + i * nwg;
    const int u = tau / NJS, js = tau - u * NJS;
    const uint8_t* base = Ld.pool + static_cast<int64_t>(M.slot[u]) * Ld.slot_bytes;
    TileRegs r;
    tile_load<FMT, UPW>(r, base, lay.G, R, 64 * static_cast<int64_t>(js) + lane, wave, nu);
    for (uint32_t mask = M.mask[u]; mask != 0u; mask &= mask - 1u) {
      const int t = __builtin_ctz(mask);
      const float row = tile_row<FMT, UPW>(r, xl + static_cast<int64_t>(t) * d, bsum[t], wave, nu);
      red[wave][lane] = row;
      __syncthreads();
      if (wave == 0) {
        float rs = red[0][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) rs += red[w][lane];
        // up row 2j+1 sits in the lane after gate row 2j
        const float up = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, rs), 0xB1, 0xF, 0xF, false));
        const float hv = silu(rs) * up;
        if ((lane & 1) == 0)
          store_agent(hl + (static_cast<int64_t>(u) * T + t) * f + TILE_H * js + (lane >> 1), hv);
      }
      __syncthreads();
    }
  }

  if (remainder && wg < left * TILE_H) {
    // one h index of a left-over tile, one lane per block (waves 0 and 1:
    // gate and up row), then the tile path's sums in the tile path's order
    const int tau = full * nwg + wg / TILE_H, jl = wg % TILE_H;
    const int u = tau / NJS, js = tau - u * NJS;
    const uint8_t* base = Ld.pool + static_cast<int64_t>(M.slot[u]) * Ld.slot_bytes;
    float(*racc)[64] = reinterpret_cast<float(*)[64]>(smem + LL.racc);
    uint32_t(*rs16)[64] = reinterpret_cast<uint32_t(*)[64]>(smem + LL.rs16);
    uint32_t(*rm16)[64] = reinterpret_cast<uint32_t(*)[64]>(smem + LL.rm16);
    float(*red2)[16] = reinterpret_cast<float(*)[16]>(smem + LL.red2);
    const int nb = d / 32;
    const int rho = wave;   // 0: gate row, 1: up row
    uint2 cc = make_uint2(0u, 0u);
    uint32_t sc = 0u, mn = 0u, hi = 0u;
    if (wave < 2) {
      const int b = min(lane, nb - 1);
      const int64_t row = 64 * static_cast<int64_t>(js) + 2 * jl + rho;
      const int64_t unit = static_cast<int64_t>(b >> 1) * R + row;
      const int half = b & 1;
      cc = nt_u2(base + lay.G.codes + unit * 16 + half * 8);
      sc = nt_u16(base + lay.G.scale + unit * 4 + half * 2);
      if (FMT == MOE_FMT_Q2SM) mn = nt_u16(base + lay.G.min + unit * 4 + half * 2);
      if (FMT == MOE_FMT_Q3G) hi = nt_u32(base + lay.G.hi + unit * 8 + half * 4);
    }
    for (uint32_t mask = M.mask[u]; mask != 0u; mask &= mask - 1u) {
      const int t = __builtin_ctz(mask);
      if (wave < 2) {
        const int b = min(lane, nb - 1);
        const float* xt = xl + static_cast<int64_t>(t) * d + 32 * b;
        float xr[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 v = reinterpret_cast<const float4*>(xt)[q];
          xr[4 * q] = v.x;
          xr[4 * q + 1] = v.y;
          xr[4 * q + 2] = v.z;
          xr[4 * q + 3] = v.w;
        }
        const float acc = block_acc<FMT>(cc.x, cc.y, hi, xr, 0);
        if (lane < nb) {
          racc[rho][lane] = acc;
          rs16[rho][lane] = sc;
          rm16[rho][lane] = mn;
        }
      }
      __syncthreads();
      if (wave < 2 && lane < NW) {
        const float2* bs = bsum[t];
        float row = 0.0f;
#pragma unroll
        for (int i = 0; i < UPW; ++i) {
          const int c = lane + NW * i;
          if (c < nu) {
            row = block_finish<FMT>(row, racc[rho][2 * c], bs[2 * c].y, bs[2 * c].x,
                                    rs16[rho][2 * c], rm16[rho][2 * c]);
            row = block_finish<FMT>(row, racc[rho][2 * c + 1], bs[2 * c + 1].y, bs[2 * c + 1].x,
                                    rs16[rho][2 * c + 1], rm16[rho][2 * c + 1]);
          }
        }
        red2[rho][lane] = row;
      }
      __syncthreads();
      if (tid == 0) {
        float g = red2[0][0], up = red2[1][0];
        for (int w = 1; w < NW; ++w) {
          g += red2[0][w];
          up += red2[1][w];
        }
        store_agent(hl + (static_cast<int64_t>(u) * T + t) * f + TILE_H * js + jl, silu(g) * up);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// down phase
// ---------------------------------------------------------------------------

template <int FMT>
__device__ void down_phase(const StackArgs& a, const StackLayerDev& Ld, const Members& M,
                           const float* xl, const float* hl, float* xnext,
                           const float* addend_next, uint8_t* smem, const LdsLayout& LL) {
  const int tid = threadIdx.x;
  const int wg = blockIdx.x, nwg = a.nwg;
  const int d = a.d, f = a.f, T = a.T, k = a.k;
  const int NKB = f / 32;
  const int gpt = nwg / T;                 // workgroups per token
  const int t = wg / gpt;
  if (t >= T) return;
  const int ci = wg - t * gpt;
  const int rb = (d + gpt - 1) / gpt;
  const int rbeg = ci * rb, rend = min(d, rbeg + rb);
  if (rbeg >= rend) return;

  // terms of token t: chosen resident experts in k-slot order, then shared
  int* tq_mem = reinterpret_cast<int*>(smem + LL.tq);
  float* tq_w = reinterpret_cast<float*>(smem + LL.tq + MAXM * 4);
  if (tid == 0) {
    int nq = 0;
    for (int i = 0; i < k; ++i) {
      const int u = M.pm[t * k + i];
      if (u >= 0) {
        tq_mem[nq] = u;
        tq_w[nq] = M.w[t * k + i];
        ++nq;
      }
    }
    tq_mem[MAXM - 1] = nq;   // routed terms; the shared member follows if any
  }
  __syncthreads();
  const int nq_routed = tq_mem[MAXM - 1];
  const bool has_shared = M.n_m > M.n_routed;
  const int nq = nq_routed + (has_shared ? 1 : 0);
  auto term_member = [&](int q) { return q < nq_routed ? tq_mem[q] : M.n_routed; };

  const SlotLayout lay = slot_layout(FMT, d, f);
  float* bbuf = reinterpret_cast<float*>(smem + LL.b);
  float* obuf = reinterpret_cast<float*>(smem + LL.obuf);

  for (int r0 = rbeg; r0 < rend; r0 += RMAX) {
    const int nr = min(RMAX, rend - r0);
    // terms per chunk: h (f), block sums (NKB float2), parts (NKB * nr)
    const int per_term = f * 4 + NKB * 8 + NKB * nr * 4;
    const int qc = max(1, B_BUDGET / per_term);
    for (int q0 = 0; q0 < nq; q0 += qc) {
      const int q1 = min(nq, q0 + qc);
      const int nqc = q1 - q0;
      float* hs = bbuf;                                            // [nqc][f]
      float2* hk = reinterpret_cast<float2*>(bbuf + nqc * f);      // [nqc][NKB]
      float* part = bbuf + nqc * f + 2 * nqc * NKB;                // [nqc][NKB][nr]
      for (int e = tid; e < nqc * f; e += NT) {
        const int qq = e / f, j = e - qq * f;
        hs[e] = hl[(static_cast<int64_t>(term_member(q0 + qq)) * T + t) * f + j];
      }
      __syncthreads();
      for (int e = tid; e < nqc * NKB; e += NT) {
        const float* h = hs + e * 32;   // (qq, kb) -> h block (qq*f + 32kb = 32e)
        float hx = 0.0f, hc = 0.0f;
#pragma unroll 8
        for (int j = 0; j < 32; ++j) {
          hx += h[j];
          hc = fmaf(block_offset_weight<FMT>(j), h[j], hc);
        }
        hk[e] = make_float2(hx, block_const<FMT>(hx, hc));
      }
      __syncthreads();
      const int n_it = nqc * NKB * nr;
      for (int it = tid; it < n_it; it += NT) {
        const int r = it % nr;
        const int rest = it / nr;
        const int kb = rest % NKB, qq = rest / NKB;
        const int u = term_member(q0 + qq);
        const uint8_t* base = Ld.pool + static_cast<int64_t>(M.slot[u]) * Ld.slot_bytes;
        const int64_t unit = static_cast<int64_t>(kb) * d + r0 + r;
        const uint2 cc = nt_u2(base + lay.D.codes + unit * 8);
        const uint32_t sc = nt_u16(base + lay.D.scale + unit * 2);
        const uint32_t mn = FMT == MOE_FMT_Q2SM ? nt_u16(base + lay.D.min + unit * 2) : 0u;
        const uint32_t hi = FMT == MOE_FMT_Q3G ? nt_u32(base + lay.D.hi + unit * 4) : 0u;
        float hv[32];
        const float4* hp = reinterpret_cast<const float4*>(hs + qq * f + 32 * kb);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float4 v = hp[q];
          hv[4 * q] = v.x;
          hv[4 * q + 1] = v.y;
          hv[4 * q + 2] = v.z;
          hv[4 * q + 3] = v.w;
        }
        const float acc = block_acc<FMT>(cc.x, cc.y, hi, hv, 0);
        const float2 kk = hk[qq * NKB + kb];
        part[(qq * NKB + kb) * nr + r] = block_finish<FMT>(0.0f, acc, kk.y, kk.x, sc, mn);
      }
      __syncthreads();
      for (int e = tid; e < nqc * nr; e += NT) {
        const int qq = e / nr, r = e - qq * nr;
        float o = part[(qq * NKB) * nr + r];
        for (int kb = 1; kb < NKB; ++kb) o += part[(qq * NKB + kb) * nr + r];
        obuf[(q0 + qq) * RMAX + r] = o;
      }
      __syncthreads();
    }
    // y = x + sum_i w_i o_i (k-slot order) + o_shared
    for (int r = tid; r < nr; r += NT) {
      const int64_t o = static_cast<int64_t>(t) * d + r0 + r;
      float acc = xl[o];
      for (int q = 0; q < nq_routed; ++q) acc = fmaf(tq_w[q], obuf[q * RMAX + r], acc);
      if (has_shared) acc += obuf[nq_routed * RMAX + r];
      if (Ld.y) Ld.y[o] = acc;
      if (xnext) {
        const float xn = addend_next ? acc + addend_next[o] : acc;
        store_agent(xnext + o, xn);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

template <int UPW>
__global__ __launch_bounds__(NT) void decode_stack_kernel(StackArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr LdsLayout LL = lds_layout();
  Members* mem = reinterpret_cast<Members*>(smem + LL.mem);
  const int wg = blockIdx.x;
  const unsigned gen = a.sync[SY_GEN];
  unsigned bar = 0;
  auto epoch = [&](unsigned b) { return gen * 64u + b + 1u; };
  const bool pairs = a.pairs_mode != 0;

  stack_route(a, a.L[0], pairs, smem, LL, mem[0]);
  for (int l = 0; l < a.n_layers; ++l) {
    const StackLayerDev& Ld = a.L[l];
    Members& M = mem[l & 1];
    if (l > 0) {
      bar_wait(a.sync, epoch(bar));   // barrier Y of layer l-1
      ++bar;
      if (a.route_after_x) stack_route(a, Ld, false, smem, LL, M);
    }
    const float* xl = l == 0 ? a.x0 : a.xbuf + l * a.x_stride;
    float* hl = a.hbuf + l * a.h_stride;
    switch (Ld.fmt) {
      case MOE_FMT_Q2S: gateup_phase<MOE_FMT_Q2S, UPW>(a, Ld, M, xl, hl, smem, LL); break;
      case MOE_FMT_Q2SM: gateup_phase<MOE_FMT_Q2SM, UPW>(a, Ld, M, xl, hl, smem, LL); break;
      default: gateup_phase<MOE_FMT_Q3G, UPW>(a, Ld, M, xl, hl, smem, LL); break;
    }
    bar_arrive(a.sync, wg, a.nwg, epoch(bar));   // barrier H
    if (!a.route_after_x && l + 1 < a.n_layers)
      stack_route(a, a.L[l + 1], false, smem, LL, mem[(l + 1) & 1]);
    bar_wait(a.sync, epoch(bar));
    ++bar;
    const bool last = l + 1 == a.n_layers;
    float* xnext = last ? a.xout : a.xbuf + (l + 1) * a.x_stride;
    const float* addend_next = last ? a.addend_next : a.L[l + 1].addend;
    switch (Ld.fmt) {
      case MOE_FMT_Q2S:
        down_phase<MOE_FMT_Q2S>(a, Ld, M, xl, hl, xnext, addend_next, smem, LL);
        break;
      case MOE_FMT_Q2SM:
        down_phase<MOE_FMT_Q2SM>(a, Ld, M, xl, hl, xnext, addend_next, smem, LL);
        break;
      default:
        down_phase<MOE_FMT_Q3G>(a, Ld, M, xl, hl, xnext, addend_next, smem, LL);
        break;
    }
    if (!last) bar_arrive(a.sync, wg, a.nwg, epoch(bar));   // barrier Y
  }
  if (wg == 0 && threadIdx.x == 0) a.sync[SY_GEN] = gen + 1u;
}

}  // namespace

size_t stack_sync_bytes() { return 2048; }

size_t decode_stack_workspace_bytes(int d, int f, int T, int k, int n_layers) {
  const int per_launch = n_layers < MOE_MAX_STACK_LAYERS ? n_layers : MOE_MAX_STACK_LAYERS;
  const int64_t h = align256(static_cast<int64_t>(T * k + 1) * T * f * 4);
  const int64_t x = align256(static_cast<int64_t>(T) * d * 4) + 4096;   // guard between layers
  return stack_sync_bytes() + static_cast<size_t>(align256(static_cast<int64_t>(T) * d * 4)) +
         static_cast<size_t>(per_launch) * static_cast<size_t>(h + x);
}

hipError_t launch_decode_stack(const StackDims& D, int n_layers, const moe_stack_layer* layers,
                               const float* x, const int32_t* in_idx, const int32_t* in_slot,
                               const float* in_w, int flags, void* ws, hipStream_t s) {
  int dev = 0, n_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int per_launch = n_layers < MOE_MAX_STACK_LAYERS ? n_layers : MOE_MAX_STACK_LAYERS;
  uint8_t* p = static_cast<uint8_t*>(ws);
  unsigned* sync = reinterpret_cast<unsigned*>(p);
  p += stack_sync_bytes();
  float* xcarry = reinterpret_cast<float*>(p);
  p += align256(static_cast<int64_t>(D.T) * D.d * 4);
  const int64_t h_bytes = align256(static_cast<int64_t>(D.T * D.k + 1) * D.T * D.f * 4);
  const int64_t x_bytes = align256(static_cast<int64_t>(D.T) * D.d * 4) + 4096;
  float* hbuf = reinterpret_cast<float*>(p);
  p += per_launch * h_bytes;
  float* xbuf = reinterpret_cast<float*>(p);

  const void* kern = D.d / 64 <= NW ? reinterpret_cast<const void*>(&decode_stack_kernel<1>)
                                    : reinterpret_cast<const void*>(&decode_stack_kernel<2>);
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, STACK_LDS);
  if (e != hipSuccess) return e;

  for (int l0 = 0; l0 < n_layers; l0 += MOE_MAX_STACK_LAYERS) {
    const int nl = n_layers - l0 < MOE_MAX_STACK_LAYERS ? n_layers - l0 : MOE_MAX_STACK_LAYERS;
    StackArgs a = {};
    a.d = D.d;
    a.f = D.f;
    a.E = D.E;
    a.k = D.k;
    a.T = D.T;
    a.n_layers = nl;
    a.route_after_x = (flags & MOE_STACK_ROUTE_AFTER_X) ? 1 : 0;
    a.pairs_mode = in_slot ? 1 : 0;
    a.nwg = n_cu;
    a.x0 = l0 == 0 ? x : xcarry;
    const bool more = l0 + nl < n_layers;
    a.xout = more ? xcarry : nullptr;
    a.addend_next = more ? layers[l0 + nl].addend : nullptr;
    a.sync = sync;
    a.hbuf = hbuf;
    a.h_stride = h_bytes / 4;
    a.xbuf = xbuf;
    a.x_stride = x_bytes / 4;
    a.in_idx = in_idx;
    a.in_slot = in_slot;
    a.in_w = in_w;
    for (int i = 0; i < nl; ++i) {
      const moe_stack_layer& S = layers[l0 + i];
      StackLayerDev& Ld = a.L[i];
      Ld.pool = static_cast<const uint8_t*>(S.pool);
      Ld.slot_bytes = S.slot_bytes;
      Ld.table = S.slot_of_expert;
      Ld.logits = S.logits;
      Ld.addend = S.addend;
      Ld.y = S.y;
      Ld.idx = S.idx;
      Ld.w = S.w;
      Ld.slot = S.slot;
      Ld.miss_expert = S.miss_expert;
      Ld.miss_pair = S.miss_pair;
      Ld.n_miss = S.n_miss;
      Ld.n_slots = S.n_slots;
      Ld.fmt = S.fmt;
      Ld.shared_slot = S.shared_slot;
    }
    void* kargs[] = {&a};
    e = hipLaunchCooperativeKernel(kern, dim3(n_cu), dim3(NT), kargs, STACK_LDS, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bitffn
