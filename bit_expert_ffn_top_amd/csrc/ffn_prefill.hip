// Prefill chunk: tokens grouped by expert, two grouped GEMMs on bf16 MFMA.
//
// 1. group: the hit pairs are counting-sorted by expert id (stable in (t, i));
//    expert_offsets, pair_pos and the permutation come out of it, plus the
//    prefix sums of each group's number of 128-row tiles.  The shared
//    expert is one more group holding all T tokens.
// 2. gate/up GEMM: for a tile of 128 rows of one group and 64 h indices, the
//    128 matching G rows (gate and up of the same h indices) are dequantized
//    to bf16 in LDS, the token rows are gathered from x by the permutation,
//    and v_mfma_f32_32x32x16_bf16 accumulates in fp32.  Each wavefront owns a
//    64 x 64 quarter; its two 32-column MFMA tiles hold gate and up of the
//    same h indices, so h = silu(g) * u is formed in registers, rounded to
//    bf16 and stored in group order.
// 3. down GEMM: the same machinery on h x D^T writes fp32 rows, per pair in
//    group order (out_pairs) or per token for the shared expert.
// The weight tiles are the only place the packed bytes are read; a tile is
// dequantized once per 128 rows of its group.
#include "moe_internal.h"

namespace bitffn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (padding vs bank conflicts)

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
  ti.m0 = (mt - g.tile_base[lo]) * BM;
  if (lo < g.E) {
    const int start = g.offsets[lo];
    const int n = g.offsets[lo + 1] - start;
    ti.rows = min(BM, n - ti.m0);
    ti.slot = g.slot[g.perm[start]];
    ti.row_base = start;
  } else {
    ti.rows = min(BM, g.T - ti.m0);
    ti.slot = g.shared_slot;
    ti.row_base = g.T * g.k;
  }
  return ti;
}

// token of local row m of the tile's group
__device__ __forceinline__ int tile_token(const GroupInfo& g, const TileInfo& ti, int m) {
  if (ti.group < g.E) return g.perm[ti.row_base + m] / g.k;
  return m;
}

// Bit of a block's 32-bit hi word that holds bit 2 of code j.
__device__ __forceinline__ int hi_bit(int j) { return j < 16 ? 2 * j + 1 : 2 * (j - 16); }

// Dequantize one 32-weight block (codes at byte offset oc, scale at os, min at
// om, hi word at oh, all from `base`) to bf16 and store 64 bytes at dst.
template <int FMT>
__device__ __forceinline__ void dequant_block_to_lds(const uint8_t* base, int64_t oc, int64_t os,
                                                     int64_t om, int64_t oh, __bf16* dst) {
  const uint2 cw = *reinterpret_cast<const uint2*>(base + oc);
  const float s = half_bits_to_float(*reinterpret_cast<const uint16_t*>(base + os));
  float m = 0.0f;
  uint32_t hi = 0;
  if (FMT == MOE_FMT_Q2SM) m = half_bits_to_float(*reinterpret_cast<const uint16_t*>(base + om));
  if (FMT == MOE_FMT_Q3G) hi = *reinterpret_cast<const uint32_t*>(base + oh);
  uint32_t packed[16];
#pragma unroll
  for (int j = 0; j < 32; j += 2) {
    const uint32_t word = j < 16 ? cw.x : cw.y;
    const int sh = 2 * (j & 15);
    uint32_t q0 = (word >> sh) & 3u;
    uint32_t q1 = (word >> (sh + 2)) & 3u;
    if (FMT == MOE_FMT_Q3G) {
      q0 |= ((hi >> hi_bit(j)) & 1u) << 2;
      q1 |= ((hi >> hi_bit(j + 1)) & 1u) << 2;
    }
    const uint32_t b0 = float_to_bf16_rne(dequant_one<FMT>(q0, s, m));
    const uint32_t b1 = float_to_bf16_rne(dequant_one<FMT>(q1, s, m));
    packed[j >> 1] = b0 | (b1 << 16);
  }
  uint4* d4 = reinterpret_cast<uint4*>(dst);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d4[q] = make_uint4(packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]);
}

// GATEUP: A = gathered x rows (bf16 [T][d]), B = G rows, epilogue silu(g)*u -> H bf16.
// !GATEUP: A = H rows of the group, B = D rows, epilogue fp32 rows.
template <int FMT, bool GATEUP>
__global__ __launch_bounds__(256) void prefill_gemm_kernel(
    const uint8_t* __restrict__ pool, int64_t slot_bytes, Planes P, int d, int f, GroupInfo g,
    const uint16_t* __restrict__ a_src, uint16_t* __restrict__ h_out,
    float* __restrict__ out_pairs, float* __restrict__ out_shared) {
  __shared__ __attribute__((aligned(16))) __bf16 As[BM * LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) __bf16 Bs[BN * LDS_STRIDE];

  const int K = GATEUP ? d : f;              // reduction length
  const int N = GATEUP ? 2 * f : d;          // output columns of the tile space
  const int n_tiles = N / BN;
  const int total = g.tile_base[g.E + 1] * n_tiles;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int mt = tile / n_tiles;
    const int nt = tile - mt * n_tiles;
    const TileInfo ti = find_tile(g, mt);
    if (ti.slot < 0) continue;  // cannot happen for hit groups; shared slot checked on host
    const uint8_t* base = pool + static_cast<int64_t>(ti.slot) * slot_bytes;

    // A row source for this thread's load slot
    const int a_row = tid >> 1, a_half = tid & 1;
    const bool a_valid = a_row < ti.rows;
    int64_t a_off = 0;
    if (a_valid) {
      if (GATEUP)
        a_off = static_cast<int64_t>(tile_token(g, ti, ti.m0 + a_row)) * d;
      else
        a_off = static_cast<int64_t>(ti.row_base + ti.m0 + a_row) * f;
    }
    // B row of this thread's dequant slot
    const int b_n = tid >> 1, b_blk = tid & 1;
    int64_t b_row;
    if (GATEUP) {
      const int jj = (b_n & 31) + 32 * (b_n >> 6);
      const int is_up = (b_n >> 5) & 1;
      b_row = 2 * (static_cast<int64_t>(nt) * 64 + jj) + is_up;
    } else {
      b_row = static_cast<int64_t>(nt) * BN + b_n;
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += BK) {
      // A tile: 128 rows x 64 bf16, 64 B per thread
      {
        uint4 v[4];
        if (a_valid) {
          const uint4* src = reinterpret_cast<const uint4*>(a_src + a_off + k0 + 32 * a_half);
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = src[q];
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = make_uint4(0, 0, 0, 0);
        }
        uint4* dst = reinterpret_cast<uint4*>(As + a_row * LDS_STRIDE + 32 * a_half);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = v[q];
      }
      // B tile: 128 rows x 2 blocks, one block per thread.  G is stored in
      // units of 2 blocks, D in units of 1 block; unit c of row r at c*rows + r.
      {
        int64_t oc, os, om, oh;
        if (GATEUP) {
          const int64_t unit = static_cast<int64_t>(k0 / 64) * (2 * static_cast<int64_t>(f)) + b_row;
          oc = P.codes + unit * 16 + 8 * b_blk;
          os = P.scale + unit * 4 + 2 * b_blk;
          om = P.min + unit * 4 + 2 * b_blk;
          oh = P.hi + unit * 8 + 4 * b_blk;
        } else {
          const int64_t unit = static_cast<int64_t>(k0 / 32 + b_blk) * d + b_row;
          oc = P.codes + unit * 8;
          os = P.scale + unit * 2;
          om = P.min + unit * 2;
          oh = P.hi + unit * 4;
        }
        dequant_block_to_lds<FMT>(base, oc, os, om, oh, Bs + b_n * LDS_STRIDE + 32 * b_blk);
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int kofs = 16 * kk + 8 * (lane >> 5);
        bf16x8 a[2], b[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int row = 64 * wm + 32 * i + (lane & 31);
          a[i] = *reinterpret_cast<const bf16x8*>(As + row * LDS_STRIDE + kofs);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = 64 * wn + 32 * j + (lane & 31);
          b[j] = *reinterpret_cast<const bf16x8*>(Bs + col * LDS_STRIDE + kofs);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      __syncthreads();
    }

    // epilogue
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 64 * wm + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m >= ti.rows) continue;
        const int64_t orow = ti.row_base + ti.m0 + m;
        if (GATEUP) {
          const int jj = 32 * wn + (lane & 31);
          const float gv = acc[i][0][r];
          const float uv = acc[i][1][r];
          h_out[orow * f + static_cast<int64_t>(nt) * 64 + jj] = float_to_bf16_rne(silu(gv) * uv);
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int64_t col = static_cast<int64_t>(nt) * BN + 64 * wn + 32 * j + (lane & 31);
            if (ti.group < g.E)
              out_pairs[orow * d + col] = acc[i][j][r];
            else
              out_shared[static_cast<int64_t>(ti.m0 + m) * d + col] = acc[i][j][r];
          }
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

int grid_for(int64_t max_tiles) {
  const int64_t cap = 2048;
  return static_cast<int>(max_tiles < cap ? (max_tiles > 0 ? max_tiles : 1) : cap);
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
  // upper bound on m-tiles: every group rounds up once
  const int64_t max_mt = (static_cast<int64_t>(T) * L.top_k + BM - 1) / BM + L.n_experts +
                         (out_shared ? (T + BM - 1) / BM : 0);
  if (!out_shared) {
    // no shared group: make its tile count zero by treating T rows as absent
    g.shared_slot = -1;
  }
  prefill_gemm_kernel<FMT, true><<<grid_for(max_mt * (2 * L.d_ff / BN)), 256, 0, s>>>(
      static_cast<const uint8_t*>(L.pool), L.slot_bytes, lay.G, L.d_model, L.d_ff, g, x, w.h,
      nullptr, nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prefill_gemm_kernel<FMT, false><<<grid_for(max_mt * (L.d_model / BN)), 256, 0, s>>>(
      static_cast<const uint8_t*>(L.pool), L.slot_bytes, lay.D, L.d_model, L.d_ff, g, w.h,
      nullptr, out_pairs, out_shared);
  return hipGetLastError();
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
                                    w.tile_base, BM, s);
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
