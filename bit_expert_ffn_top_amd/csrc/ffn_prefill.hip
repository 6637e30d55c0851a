// Prefill chunk: tokens grouped by expert, two grouped GEMMs on bf16 MFMA.
//
// 1. group: the hit pairs are counting-sorted by expert id (stable in (t, i));
//    expert_offsets, pair_pos and the permutation come out of it, plus the
//    prefix sums of each group's number of 128-row tiles.  The shared
//    expert is one more group holding all T tokens.
// 2. gate/up GEMM, one job per (group rows, up to 256; 128 h indices): the
//    256 matching G rows (gate and up of the same h indices) are dequantized
//    to bf16 in LDS, the token rows are gathered from x by the permutation,
//    and v_mfma_f32_32x32x16_bf16 accumulates in fp32.  Four wavefronts, one
//    per SIMD: wavefront wn owns the 64 columns of h block wn and every row
//    tile (32 rows each; tiles past the group's rows are skipped by all four
//    alike); its two 32-column MFMA tiles hold gate and up of the same h
//    indices, so h = silu(g) * u is formed in registers, rounded to bf16 and
//    stored in group order.
// 3. down GEMM: the same machinery on h x D^T writes fp32 rows, per pair in
//    group order (out_pairs) or per token for the shared expert.
// Both GEMMs double-buffer the LDS tiles: the next step's x rows and packed
// blocks are loaded and dequantized while the current step's MFMAs run, with
// one barrier per step.  A routed expert's rows fit one job, so each weight
// is dequantized once per layer (the shared expert once per 256 tokens).
// Jobs are handed out persistently, all column slices of one group on the
// same XCD (job j runs on workgroup j mod grid, and workgroups are spread
// over the 8 XCDs in turn), so the gathered x rows are shared through that
// XCD's L2.
#include "moe_internal.h"

namespace bitffn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // native 16-byte vector

// A job: up to PM rows of one group (all rows of a routed expert's group in
// practice) times PN output columns, reduced in steps of PK.
constexpr int PM = 256;                  // rows (8 MFMA row tiles of 32)
constexpr int PN = 128;                  // output columns
constexpr int PK = 64;                   // reduction step
constexpr int PS = PK + 8;               // LDS row stride in bf16 (padding against bank conflicts)
constexpr int PTHREADS = 256;            // 4 wavefronts; two workgroups share a CU

struct GroupInfo {
  const int32_t* offsets;    // [E+1]
  const int32_t* perm;       // [T*k]
  const int32_t* tile_base;  // [E+2]
  const int32_t* slot;       // [T*k] slot of each pair
  int E, T, k, shared_slot;
};

// Group of flat m-tile index mt (binary search over tile_base), its row
// count, first local row, slot, and the row offset of its rows in H / out.
struct TileInfo {
  int group, m0, rows, slot, row_base;
};

__device__ __forceinline__ TileInfo find_tile(const GroupInfo& g, int mt) {
  int lo = 0, hi = g.E + 1;  // tile_base[lo] <= mt < tile_base[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (g.tile_base[mid] <= mt)
      lo = mid;
    else
      hi = mid;
  }
  TileInfo ti;
  ti.group = lo;
  ti.m0 = (mt - g.tile_base[lo]) * PM;
  if (lo < g.E) {
    const int start = g.offsets[lo];
    const int n = g.offsets[lo + 1] - start;
    ti.rows = min(PM, n - ti.m0);
    ti.slot = g.slot[g.perm[start]];
    ti.row_base = start;
  } else {
    ti.rows = min(PM, g.T - ti.m0);
    ti.slot = g.shared_slot;
    ti.row_base = g.T * g.k;
  }
  return ti;
}

// token of local row m of the tile's group (the load is unconditional, with a
// clamped index, so that the loads of several rows are issued together)
__device__ __forceinline__ int tile_token(const GroupInfo& g, const TileInfo& ti, int m) {
  const int p = g.perm[min(ti.row_base + m, g.T * g.k - 1)];
  return ti.group < g.E ? p / g.k : m;
}

// silu(z) = z / (1 + e^-z) with the hardware exponential and reciprocal
// (a few ulp in fp32, far below the bf16 rounding that follows).
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Two fp32 values rounded to bfloat16 (nearest even, one hardware
// conversion on gfx950), packed low = a, high = b.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  const bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// Bit of a block's 32-bit hi word that holds bit 2 of code j.
__device__ __forceinline__ int hi_bit(int j) { return j < 16 ? 2 * j + 1 : 2 * (j - 16); }

// Raw bytes of one 32-weight block, loaded ahead of their use.
struct BlockRaw {
  uint2 codes;
  uint32_t scale, min, hi;
};

template <int FMT>
__device__ __forceinline__ BlockRaw load_block(const uint8_t* base, int64_t oc, int64_t os,
                                               int64_t om, int64_t oh) {
  BlockRaw r;
  r.codes = *reinterpret_cast<const uint2*>(base + oc);
  r.scale = *reinterpret_cast<const uint16_t*>(base + os);
  r.min = FMT == MOE_FMT_Q2SM ? *reinterpret_cast<const uint16_t*>(base + om) : 0u;
  r.hi = FMT == MOE_FMT_Q3G ? *reinterpret_cast<const uint32_t*>(base + oh) : 0u;
  return r;
}

// The block's 32 weights (dequant_one, rounded to bf16 nearest even) as 64
// bytes at dst.
template <int FMT>
__device__ __forceinline__ void store_block_bf16(const BlockRaw& r, __bf16* dst) {
  const float s = half_bits_to_float(r.scale);
  const float m = half_bits_to_float(r.min);
  uint32_t packed[16];
#pragma unroll
  for (int j = 0; j < 32; j += 2) {
    const uint32_t word = j < 16 ? r.codes.x : r.codes.y;
    const int sh = 2 * (j & 15);
    uint32_t q0 = (word >> sh) & 3u;
    uint32_t q1 = (word >> (sh + 2)) & 3u;
    if (FMT == MOE_FMT_Q3G) {
      q0 |= ((r.hi >> hi_bit(j)) & 1u) << 2;
      q1 |= ((r.hi >> hi_bit(j + 1)) & 1u) << 2;
    }
    packed[j >> 1] = pack_bf16x2(dequant_one<FMT>(q0, s, m), dequant_one<FMT>(q1, s, m));
  }
  u32x4* d4 = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d4[q] = u32x4{packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]};
}

// One step's global loads, held in registers while the step before it is
// multiplied.  A: the step's 64 bf16 of 8 tile rows, 32*i + t/8 for i = 0..7,
// chunk t%8 of 16 bytes each (eight consecutive lanes read one 128-byte row
// piece).  B: one packed block, block t%2 of tile row t/2.
struct StepRegs {
  u32x4 a[8];
  BlockRaw b;
};

template <int FMT, bool GATEUP>
__device__ __forceinline__ void load_step(StepRegs& r, const uint16_t* __restrict__ a_src,
                                          const uint32_t (&a_off)[8], int ch, int ks,
                                          const uint8_t* __restrict__ base, const Planes& P,
                                          int64_t b_row, int bb, int d, int f) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    r.a[i] = *reinterpret_cast<const u32x4*>(a_src + a_off[i] + ks * PK + 8 * ch);
  if (GATEUP) {   // G: units of 2 blocks, unit c of row r at c * 2f + r
    const int64_t unit = static_cast<int64_t>(ks) * (2 * static_cast<int64_t>(f)) + b_row;
    r.b = load_block<FMT>(base, P.codes + unit * 16 + 8 * bb, P.scale + unit * 4 + 2 * bb,
                          P.min + unit * 4 + 2 * bb, P.hi + unit * 8 + 4 * bb);
  } else {        // D: units of 1 block, unit c of row r at c * d + r
    const int64_t unit = static_cast<int64_t>(2 * ks + bb) * d + b_row;
    r.b = load_block<FMT>(base, P.codes + unit * 8, P.scale + unit * 2, P.min + unit * 2,
                          P.hi + unit * 4);
  }
}

template <int FMT>
__device__ __forceinline__ void store_step(const StepRegs& r, __bf16* As, __bf16* Bs, int tid) {
  const int ar = tid >> 3, ch = tid & 7;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4*>(As + (32 * i + ar) * PS + 8 * ch) = r.a[i];
  store_block_bf16<FMT>(r.b, Bs + (tid >> 1) * PS + 32 * (tid & 1));
}

// MFMAs of one step for a wavefront holding row tiles rh + 2i, i < nt, and
// the two 32-column tiles at column 64*chf of the job.  All fragments of a
// 16-wide sub-step are read first (reads of unused row tiles stay inside the
// LDS tile), then the MFMAs of the used tiles run.
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[4][2], const __bf16* As, const __bf16* Bs,
                                          int lane, int rh, int chf, int nt) {
  const __bf16* a0 = As + (32 * rh + (lane & 31)) * PS + 8 * (lane >> 5);
  const __bf16* b0 = Bs + (64 * chf + (lane & 31)) * PS + 8 * (lane >> 5);
#pragma unroll
  for (int kk = 0; kk < PK / 16; ++kk) {
    const bf16x8 bv0 = *reinterpret_cast<const bf16x8*>(b0 + 16 * kk);
    const bf16x8 bv1 = *reinterpret_cast<const bf16x8*>(b0 + 32 * PS + 16 * kk);
    bf16x8 av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      av[i] = *reinterpret_cast<const bf16x8*>(a0 + 64 * i * PS + 16 * kk);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nt) {   // uniform
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv1, acc[i][1], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// GATEUP: A = gathered x rows (bf16 [T][d]), B = G rows, epilogue silu(g)*u -> H bf16.
// !GATEUP: A = H rows of the group, B = D rows, epilogue fp32 rows.
template <int FMT, bool GATEUP>
__global__ __launch_bounds__(PTHREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void
prefill_gemm_kernel(const uint8_t* __restrict__ pool, int64_t slot_bytes, Planes P, int d, int f,
                    GroupInfo g, const uint16_t* __restrict__ a_src, uint16_t* __restrict__ h_out,
                    float* __restrict__ out_pairs, float* __restrict__ out_shared) {
  __shared__ __attribute__((aligned(16))) __bf16 As[PM * PS];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[PN * PS];
  const int K = GATEUP ? d : f;              // reduction length
  const int N = GATEUP ? 2 * f : d;          // output columns of the job space
  const int nK = K / PK;
  const int n_slices = (N + PN - 1) / PN;
  const int n_gm = g.tile_base[g.E + 1];     // (group, 256-row chunk) items
  const int total = ((n_gm + 7) / 8) * 8 * n_slices;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chf = wave & 1;                  // column half: 64 columns, two MFMA tiles
  const int rh = wave >> 1;                  // row tiles rh, rh + 2, rh + 4, rh + 6

  for (int job = blockIdx.x; job < total; job += gridDim.x) {
    const int q = job >> 3;
    const int ns = q % n_slices;
    const int gm = (q / n_slices) * 8 + (job & 7);
    if (gm >= n_gm) continue;                // uniform: a padding job
    const TileInfo ti = find_tile(g, gm);
    if (ti.slot < 0) continue;               // the shared group when no shared output is wanted
    const uint8_t* __restrict__ base = pool + static_cast<int64_t>(ti.slot) * slot_bytes;
    const int rows = ti.rows;
    const int row_tiles = (rows + 31) >> 5;
    const int nt = min(4, max(0, (row_tiles - rh + 1) >> 1));   // this wavefront's row tiles

    // the 8 A rows this thread loads (clamped: rows past the group's end are
    // loaded but never stored), as element offsets; its B tile row and block
    uint32_t a_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ar = min(32 * i + (tid >> 3), rows - 1);
      a_off[i] = GATEUP ? static_cast<uint32_t>(tile_token(g, ti, ti.m0 + ar)) * d
                        : static_cast<uint32_t>(ti.row_base + ti.m0 + ar) * f;
    }
    const int ch = tid & 7;
    const int br = tid >> 1, bb = tid & 1;
    int64_t b_row;
    if (GATEUP) {   // B rows: [gate h0..31 | up h0..31 | gate h32..63 | up h32..63]
      const int h = min(ns * (PN / 2) + (br >> 6) * 32 + (br & 31), f - 1);
      b_row = 2 * static_cast<int64_t>(h) + ((br >> 5) & 1);
    } else {
      b_row = min(ns * PN + br, d - 1);
    }
    const bool cols_ok = GATEUP ? (ns * (PN / 2) + chf * 32 < f) : (ns * PN + chf * 64 < d);

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Step ks+1 is loaded into registers while step ks is multiplied; the
    // other workgroup on the CU fills the gaps at the two barriers.
    StepRegs R;
    load_step<FMT, GATEUP>(R, a_src, a_off, ch, 0, base, P, b_row, bb, d, f);
    store_step<FMT>(R, As, Bs, tid);
    __syncthreads();
    for (int ks = 0; ks < nK; ++ks) {
      const bool more = ks + 1 < nK;
      if (more) load_step<FMT, GATEUP>(R, a_src, a_off, ch, ks + 1, base, P, b_row, bb, d, f);
      if (cols_ok) {
        mfma_step(acc, As, Bs, lane, rh, chf, nt);
      }
      __syncthreads();
      if (more) {
        store_step<FMT>(R, As, Bs, tid);
        __syncthreads();
      }
    }

    // epilogue: accumulator element r of lane l holds row 8(r/4) + 4(l/32) + r%4
    // and column l%32 of its 32 x 32 tile
    if (cols_ok) {
      // row stride of the output and this lane's row base, hidden from the
      // optimizer per job so that per-element offsets are not hoisted out of
      // the job loop
      uint32_t ld = GATEUP ? f : d;
      int mlane = 4 * (lane >> 5);
      opaque(ld);
      opaque(mlane);
      uint16_t* hdst = nullptr;
      float* odst = nullptr;
      if (GATEUP) {
        hdst = h_out + static_cast<int64_t>(ti.row_base + ti.m0) * f + ns * (PN / 2) + 32 * chf +
               (lane & 31);
      } else {
        odst = (ti.group < g.E ? out_pairs + static_cast<int64_t>(ti.row_base + ti.m0) * d
                               : out_shared + static_cast<int64_t>(ti.m0) * d) +
               static_cast<int64_t>(ns) * PN + 64 * chf + (lane & 31);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nt) continue;   // uniform
        const int rt = rh + 2 * i;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * rt + 8 * (r >> 2) + (r & 3) + mlane;
          if (m < rows) {
            if (GATEUP) {
              hdst[static_cast<uint32_t>(m) * ld] =
                  float_to_bf16_rne(silu_fast(acc[i][0][r]) * acc[i][1][r]);
            } else {
              odst[static_cast<uint32_t>(m) * ld] = acc[i][0][r];
              odst[static_cast<uint32_t>(m) * ld + 32] = acc[i][1][r];
            }
          }
          if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }
}

struct PrefillWs {
  GroupWorkspace gws;
  int32_t* perm;
  int32_t* tile_base;
  uint16_t* h;
};

PrefillWs prefill_ws(void* ws, int d, int f, int T, int k, int E) {
  (void)d;
  char* p = static_cast<char*>(ws);
  PrefillWs w;
  w.gws = group_workspace(p, T, E);
  p += group_workspace_bytes(T, E);
  w.perm = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<int64_t>(T) * k * 4);
  w.tile_base = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<int64_t>(E + 2) * 4);
  w.h = reinterpret_cast<uint16_t*>(p);
  (void)f;
  return w;
}

// Persistent grid: two workgroups per CU, a multiple of 8 so that job j and
// workgroup j mod grid share an XCD.
int prefill_grid(int64_t max_jobs) {
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
      n_cu = 256;
    else
      n_cu = prop.multiProcessorCount;
  }
  int64_t grid = (max_jobs + 7) / 8 * 8;
  const int64_t cap = (2 * n_cu + 7) / 8 * 8;
  if (grid > cap) grid = cap;
  return static_cast<int>(grid > 8 ? grid : 8);
}

template <int FMT, bool GATEUP>
hipError_t launch_gemm(const GroupInfo& g, int64_t max_jobs, const moe_layer& L, Planes P,
                       const uint16_t* a, uint16_t* h, float* out_pairs, float* out_shared,
                       hipStream_t s) {
  prefill_gemm_kernel<FMT, GATEUP><<<prefill_grid(max_jobs), PTHREADS, 0, s>>>(
      static_cast<const uint8_t*>(L.pool), L.slot_bytes, P, L.d_model, L.d_ff, g, a, h, out_pairs,
      out_shared);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_prefill_fmt(const moe_layer& L, const uint16_t* x, int T, const int32_t* slot,
                              float* out_pairs, int32_t* expert_offsets, float* out_shared,
                              const PrefillWs& w, hipStream_t s) {
  const SlotLayout lay = slot_layout(L.fmt, L.d_model, L.d_ff);
  GroupInfo g;
  g.offsets = expert_offsets;
  g.perm = w.perm;
  g.tile_base = w.tile_base;
  g.slot = slot;
  g.E = L.n_experts;
  g.T = T;
  g.k = L.top_k;
  g.shared_slot = out_shared ? L.shared_slot : -1;
  // upper bound on (group, 256-row chunk) items: every group rounds up once
  const int64_t max_gm = (static_cast<int64_t>(T) * L.top_k + PM - 1) / PM + L.n_experts +
                         (out_shared ? (T + PM - 1) / PM : 0);
  hipError_t e = launch_gemm<FMT, true>(g, max_gm * ((2 * L.d_ff + PN - 1) / PN), L, lay.G, x,
                                        w.h, nullptr, nullptr, s);
  if (e != hipSuccess) return e;
  return launch_gemm<FMT, false>(g, max_gm * ((L.d_model + PN - 1) / PN), L, lay.D, w.h, nullptr,
                                 out_pairs, out_shared, s);
}

}  // namespace

size_t prefill_workspace_bytes(int d, int f, int T, int k, int E) {
  (void)d;
  return group_workspace_bytes(T, E) + static_cast<size_t>(align256(static_cast<int64_t>(T) * k * 4)) +
         static_cast<size_t>(align256(static_cast<int64_t>(E + 2) * 4)) +
         static_cast<size_t>(align256((static_cast<int64_t>(T) * k + T) * f * 2));
}

hipError_t launch_prefill(const moe_layer& L, const uint16_t* x_bf16, int T, const int32_t* idx,
                          const int32_t* slot, float* out_pairs, int32_t* pair_pos,
                          int32_t* expert_offsets, float* out_shared, void* ws, hipStream_t s) {
  const PrefillWs w = prefill_ws(ws, L.d_model, L.d_ff, T, L.top_k, L.n_experts);
  // a shared group with zero rows when no shared output is wanted
  const int T_shared = out_shared ? T : 0;
  hipError_t e = launch_group_pairs(idx, slot, nullptr, T, L.top_k, L.n_experts, true, w.gws,
                                    expert_offsets, w.perm, pair_pos, nullptr, nullptr,
                                    w.tile_base, PM, s);
  if (e != hipSuccess) return e;
  (void)T_shared;
  switch (L.fmt) {
    case MOE_FMT_Q2S:
      return launch_prefill_fmt<MOE_FMT_Q2S>(L, x_bf16, T, slot, out_pairs, expert_offsets,
                                             out_shared, w, s);
    case MOE_FMT_Q2SM:
      return launch_prefill_fmt<MOE_FMT_Q2SM>(L, x_bf16, T, slot, out_pairs, expert_offsets,
                                              out_shared, w, s);
    case MOE_FMT_Q3G:
      return launch_prefill_fmt<MOE_FMT_Q3G>(L, x_bf16, T, slot, out_pairs, expert_offsets,
                                             out_shared, w, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace bitffn
