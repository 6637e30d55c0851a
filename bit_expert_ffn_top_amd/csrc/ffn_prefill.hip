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
#include <atomic>

#include "moe_internal.h"

namespace bitffn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // native 16-byte vector

// A job: up to PM rows of one group (all rows of a routed expert's group in
// practice) times PN output columns, reduced in steps of PK.
constexpr int PM = 256;                  // rows: 8 MFMA tiles of 32 tokens
constexpr int PN = 256;                  // output columns: 8 MFMA tiles of 32
constexpr int PK = 64;                   // reduction step
constexpr int NCONS = 512;               // 8 MFMA wavefronts, two per SIMD
constexpr int NPROD = 256;               // 4 loading / dequantizing wavefronts, one per SIMD
constexpr int PTHREADS = NCONS + NPROD;
// LDS: three A tiles (token rows) and two B tiles (dequantized weight rows),
// 128 bytes per row (half of the 64 banks) with the 16-byte piece c of row r
// at position c ^ swz(r), swz(r) = (r % 8) ^ (r/8 % 2): the 16 consecutive rows
// that a 16-byte-per-lane LDS access serves together then fall in 16
// distinct groups of 4 banks.  160 KB: all of a CU's LDS.
constexpr int A_TILE = PM * PK;          // bf16 elements
constexpr int B_TILE = PN * PK;
constexpr int A_BUFS = 3;
constexpr size_t PREFILL_LDS = (A_BUFS * A_TILE + 2 * B_TILE) * sizeof(__bf16);

__host__ __device__ constexpr int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct GroupInfo {
  const int32_t* offsets;     // [E+1]
  const int32_t* perm;        // [T*k]
  const int32_t* tile_base;   // [E+2]
  const int32_t* tile_group;  // [tiles]: the group of every tile
  const int32_t* group_slot;  // [E]: the slot of every non-empty group
  int E, T, k, shared_slot;
};

// Group of flat m-tile index mt, its row count, first local row, slot, and
// the row offset of its rows in H / out: two levels of loads (the tile's
// group, then that group's bounds and slot).
struct TileInfo {
  int group, m0, rows, slot, row_base;
};

__device__ __forceinline__ TileInfo find_tile(const GroupInfo& g, int mt) {
  const int e = g.tile_group[mt];
  TileInfo ti;
  ti.group = e;
  ti.m0 = (mt - g.tile_base[e]) * PM;
  if (e < g.E) {
    const int start = g.offsets[e];
    ti.rows = min(PM, g.offsets[e + 1] - start - ti.m0);
    ti.slot = g.group_slot[e];
    ti.row_base = start;
  } else {
    ti.rows = min(PM, g.T - ti.m0);
    ti.slot = g.shared_slot;
    ti.row_base = g.T * g.k;
  }
  return ti;
}

// Job j of the job space: its column slice and tile; false for a padding job
// or a group with nothing to run (the shared expert without a shared output).
__device__ __forceinline__ bool fetch_job(const GroupInfo& g, int n_slices, int n_gm, int total,
                                          int job, int& ns, TileInfo& ti) {
  if (job >= total) return false;
  const int q = job >> 3;
  ns = q % n_slices;
  // tiles from the last one down: the shared expert's full 256-row tiles
  // (the longest jobs) first, so that the short ones fill the end
  const int gm = n_gm - 1 - ((q / n_slices) * 8 + (job & 7));
  if (gm < 0) return false;
  ti = find_tile(g, gm);
  return ti.slot >= 0;
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

// The block's 32 weights (dequant_one, rounded to bf16 nearest even) as four
// 16-byte pieces piece0 .. piece0+3 of a 128-byte LDS row, piece c stored at
// position c ^ key.
template <int FMT>
__device__ __forceinline__ void store_block_bf16(const BlockRaw& r, __bf16* row, int piece0,
                                                 int key) {
  const float s = half_bits_to_float(r.scale);
  const float m = half_bits_to_float(r.min);
  uint32_t packed[16];
  // Q2S: s*(q - 1.5) = s*q + (-1.5 s), -1.5 s exact
  const float m0 = FMT == MOE_FMT_Q2SM ? m : -1.5f * s;
  if (FMT != MOE_FMT_Q3G) {
    // A 2-bit code takes one of four values, w_q = fma(s, q, m0) rounded to
    // bf16 once: they form an 8-byte table (w_0 w_1 | w_2 w_3), and each pair
    // of weights is picked from it by one byte permute whose selector holds
    // bytes 2q, 2q+1 of each code (about 2 vector instructions per weight
    // instead of 2.6; the same bits as dequantizing every weight).
    const uint32_t t01 = pack_bf16x2(fmaf(s, 0.0f, m0), fmaf(s, 1.0f, m0));
    const uint32_t t23 = pack_bf16x2(fmaf(s, 2.0f, m0), fmaf(s, 3.0f, m0));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = h == 0 ? r.codes.x : r.codes.y;
      // 2q of codes 4i, 4i+1, 4i+2, 4i+3 in byte i of d0, d1, d2, d3
      const uint32_t d0 = (w << 1) & 0x06060606u, d1 = (w >> 1) & 0x06060606u;
      const uint32_t d2 = (w >> 3) & 0x06060606u, d3 = (w >> 5) & 0x06060606u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {   // weights 2j, 2j+1 of this word
        const uint32_t lo = (j & 1) ? d2 : d0, hi = (j & 1) ? d3 : d1;
        const uint32_t b = static_cast<uint32_t>(j >> 1);
        // (2q_a, 2q_a, 2q_b, 2q_b), then + 1 in the high byte of each weight
        const uint32_t sel =
            __builtin_amdgcn_perm(hi, lo, b | (b << 8) | ((4u + b) << 16) | ((4u + b) << 24)) |
            0x01000100u;
        packed[8 * h + j] = __builtin_amdgcn_perm(t23, t01, sel);
      }
    }
    u32x4* d4 = reinterpret_cast<u32x4*>(row);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      d4[(piece0 + q) ^ key] =
          u32x4{packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]};
    return;
  }
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
  u32x4* d4 = reinterpret_cast<u32x4*>(row);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    d4[(piece0 + q) ^ key] =
        u32x4{packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]};
}

// Buffer resource over `bytes` bytes at base (raw, unswizzled; gfx9 word 3).
// Loads through it take a 32-bit per-lane offset and a wave-uniform offset,
// so the per-step advance costs no vector instructions.
typedef __amdgpu_buffer_rsrc_t BufRsrc;
__device__ __forceinline__ BufRsrc buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           static_cast<int>(bytes), 0x00020000);
}

// The weight block of this thread for step ks: block vb of the step's
// blocks, whose first block index is sblk (wave-uniform).
template <int FMT, bool GATEUP>
__device__ __forceinline__ BlockRaw load_b(BufRsrc rs, const Planes& P, uint32_t vb, int ks, int d,
                                           int f) {
  // G: units of 2 blocks, unit c of row r at c * 2f + r, so step ks starts
  // at block 4f*ks; D: units of 1 block, unit c of row r at c * d + r, and a
  // step is two units
  const int64_t sblk = GATEUP ? static_cast<int64_t>(ks) * 4 * f : static_cast<int64_t>(ks) * 2 * d;
  BlockRaw r;
  // weight blocks are read once: cache policy 2 = nontemporal
  const auto c = __builtin_amdgcn_raw_buffer_load_b64(rs, vb * 8,
                                                      static_cast<int>(P.codes + sblk * 8), 2);
  r.codes = make_uint2(c[0], c[1]);
  r.scale = __builtin_amdgcn_raw_buffer_load_b16(rs, vb * 2, static_cast<int>(P.scale + sblk * 2),
                                                 2);
  r.min = FMT == MOE_FMT_Q2SM ? __builtin_amdgcn_raw_buffer_load_b16(
                                    rs, vb * 2, static_cast<int>(P.min + sblk * 2), 2)
                              : 0u;
  r.hi = FMT == MOE_FMT_Q3G
             ? __builtin_amdgcn_raw_buffer_load_b32(rs, vb * 4, static_cast<int>(P.hi + sblk * 4), 2)
             : 0u;
  return r;
}

// Producer side.  The 256 producer threads (index p, wavefront pw = p/64,
// lane l) move the token rows of a step straight from memory into an A tile:
// eight 1 KB loads per wavefront that write LDS directly, lane l's 16 bytes
// at 16*l, so load j covers tile rows 64pw + 8j .. +7 and lane l reads piece
// (l%8) ^ swz(r) of row r = 64pw + 8j + l/8 from memory (a row past the
// group's end has an offset outside the buffer, which loads zero).  They also load
// both weight blocks of tile row p and dequantize them into the B tile.
struct ProdCtx {
  BufRsrc a_rs;              // the A rows (x or H)
  BufRsrc b_rs;              // the expert's slot
  uint32_t a_voff[8];        // byte offsets of this lane's 8 row pieces
  uint32_t vb[2];            // this thread's two blocks within a step's blocks
  int p, nK;
};

template <int FMT>
constexpr int block_loads() {   // memory instructions per block
  return 2 + (FMT == MOE_FMT_Q2SM ? 1 : 0) + (FMT == MOE_FMT_Q3G ? 1 : 0);
}

__device__ __forceinline__ void load_a_lds(const ProdCtx& c, __bf16* abuf, int ks) {
  const int pw = c.p >> 6;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        c.a_rs, (__attribute__((address_space(3))) void*)(abuf + (64 * pw + 8 * j) * PK), 16,
        c.a_voff[j], ks * (PK * 2), 0, 0);
}

template <int FMT, bool GATEUP>
__device__ __forceinline__ void load_step(BlockRaw (&r)[2], const ProdCtx& c, const Planes& P,
                                          int ks, int d, int f) {
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) r[bb] = load_b<FMT, GATEUP>(c.b_rs, P, c.vb[bb], ks, d, f);
}

template <int FMT>
__device__ __forceinline__ void store_step(const BlockRaw (&r)[2], __bf16* Bs, const ProdCtx& c) {
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) store_block_bf16<FMT>(r[bb], Bs + c.p * PK, 4 * bb, swz(c.p));
}

// Wait until at most N memory instructions of this wavefront are in flight
// (they complete in order).  s_waitcnt fields: vmcnt bits 3:0 and 15:14,
// expcnt 6:4 (7: no wait), lgkmcnt 11:8 (15: no wait).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier of the GEMM steps.  It waits for this wavefront's LDS
// reads and writes (lgkmcnt 0) and for nothing else: the barrier with a
// workgroup fence also waits for every outstanding load that writes LDS (the
// rows requested for a later step) and for the epilogue's global stores, so
// that each step would pay their latency.  The loads that must have landed
// are waited for explicitly (wait_vm) by the producers before they arrive
// here.  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void step_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt: no wait
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One producer step ks: the token rows of step ks+2 are requested into the A
// buffer that step ks-1 used, the weight blocks of step ks+3 into `load`, the
// blocks of step ks+1 (`use`, requested two steps earlier) are dequantized
// into the free B buffer, and the rows of step ks+1 (requested one step
// earlier) are waited for before the barrier.  Weight loads past the last
// step repeat it (unconditional loads); the last stores of a job are repeats
// that nobody reads.
template <int FMT, bool GATEUP>
__device__ __forceinline__ void produce_step(const ProdCtx& c, const Planes& P, int d, int f,
                                             __bf16* abuf, __bf16* bbuf, int ks,
                                             const BlockRaw (&use)[2], BlockRaw (&load)[2]) {
  constexpr int NB = 2 * block_loads<FMT>();
  const bool more = ks + 2 < c.nK;
  if (more) load_a_lds(c, abuf + ((ks + 2) % A_BUFS) * A_TILE, ks + 2);
  store_step<FMT>(use, bbuf + ((ks + 1) & 1) * B_TILE, c);
  load_step<FMT, GATEUP>(load, c, P, min(ks + 3, c.nK - 1), d, f);
  // newer than the rows of step ks+1: the blocks of steps ks+2 and ks+3 and
  // the rows of step ks+2
  if (more)
    wait_vm<2 * NB + 8>();
  else
    wait_vm<2 * NB>();
  step_barrier();
}

template <int FMT, bool GATEUP>
__device__ __forceinline__ void produce_job(const ProdCtx& c, const Planes& P, int d, int f,
                                            __bf16* abuf, __bf16* bbuf) {
  constexpr int NB = 2 * block_loads<FMT>();
  BlockRaw R0[2], R1[2];
  load_a_lds(c, abuf, 0);
  load_step<FMT, GATEUP>(R0, c, P, 0, d, f);
  if (c.nK > 1) load_a_lds(c, abuf + A_TILE, 1);
  store_step<FMT>(R0, bbuf, c);
  load_step<FMT, GATEUP>(R0, c, P, min(1, c.nK - 1), d, f);
  load_step<FMT, GATEUP>(R1, c, P, min(2, c.nK - 1), d, f);
  // newer than the rows of step 0: the rows of step 1 and the blocks of
  // steps 0, 1, 2 (those of step 0 are done)
  if (c.nK > 1)
    wait_vm<3 * NB + 8>();
  else
    wait_vm<3 * NB>();
  step_barrier();
  int ks = 0;
  for (; ks + 1 < c.nK; ks += 2) {
    produce_step<FMT, GATEUP>(c, P, d, f, abuf, bbuf, ks, R0, R0);
    produce_step<FMT, GATEUP>(c, P, d, f, abuf, bbuf, ks + 1, R1, R1);
  }
  if (ks < c.nK) produce_step<FMT, GATEUP>(c, P, d, f, abuf, bbuf, ks, R0, R0);
}

// MFMAs of one step for a wavefront holding token tiles rh + 2i, i < NT, and
// the two 32-column tiles 2cq, 2cq + 1 of the job.  The weights are the MFMA's
// first operand, so that an accumulator holds 4 consecutive columns of one
// token per group of 4 registers: element r of lane l is column
// 8(r/4) + 4(l/32) + r%4 of its tile and token l%32.
template <int NT>
struct Frags {
  bf16x8 w[2];
  bf16x8 x[NT > 0 ? NT : 1];
};

// A fragment of row r (r % 16 = lane % 16 for every tile of a lane, in A and
// in B) at 16-byte piece 2kk + lane/32 sits at byte r*128 + 16*((2kk + lane/32) ^ swz(lane)).
template <int NT>
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[NT > 0 ? NT : 1][2], const __bf16* As,
                                          const __bf16* Bs, int lane, int rh, int cq) {
  const char* a0 = reinterpret_cast<const char*>(As) + (32 * rh + (lane & 31)) * (PK * 2);
  const char* b0 = reinterpret_cast<const char*>(Bs) + (64 * cq + (lane & 31)) * (PK * 2);
  const int h = lane >> 5, l7 = swz(lane & 15);
  if (NT == 4) {   // no registers to spare: fragments read per sub-step
#pragma unroll
    for (int kk = 0; kk < PK / 16; ++kk) {
      const int pc = 16 * ((2 * kk + h) ^ l7);
      Frags<NT> c;
      c.w[0] = *reinterpret_cast<const bf16x8*>(b0 + pc);
      c.w[1] = *reinterpret_cast<const bf16x8*>(b0 + 32 * (PK * 2) + pc);
#pragma unroll
      for (int i = 0; i < NT; ++i)
        c.x[i] = *reinterpret_cast<const bf16x8*>(a0 + 64 * i * (PK * 2) + pc);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.w[0], c.x[i], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.w[1], c.x[i], acc[i][1], 0, 0, 0);
      }
    }
    return;
  }
  // Fragments roll through one register set: in sub-step kk the MFMAs with
  // weight fragment 0 go first, after which it is refilled with sub-step
  // kk+1; then those with weight fragment 1, each followed by the refill of
  // its token fragment, and last weight fragment 1.  Every read has the
  // MFMAs of the other tiles to arrive.
  Frags<NT> c;
  c.w[0] = *reinterpret_cast<const bf16x8*>(b0 + 16 * (h ^ l7));
  c.w[1] = *reinterpret_cast<const bf16x8*>(b0 + 32 * (PK * 2) + 16 * (h ^ l7));
#pragma unroll
  for (int i = 0; i < NT; ++i)
    c.x[i] = *reinterpret_cast<const bf16x8*>(a0 + 64 * i * (PK * 2) + 16 * (h ^ l7));
#pragma unroll
  for (int kk = 0; kk < PK / 16; ++kk) {
    const bool next = kk + 1 < PK / 16;
    const int pn = 16 * ((2 * kk + 2 + h) ^ l7);   // piece of sub-step kk+1
#pragma unroll
    for (int i = 0; i < NT; ++i)
      acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.w[0], c.x[i], acc[i][0], 0, 0, 0);
    if (next) c.w[0] = *reinterpret_cast<const bf16x8*>(b0 + pn);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(c.w[1], c.x[i], acc[i][1], 0, 0, 0);
      if (next) c.x[i] = *reinterpret_cast<const bf16x8*>(a0 + 64 * i * (PK * 2) + pn);
    }
    if (next) c.w[1] = *reinterpret_cast<const bf16x8*>(b0 + 32 * (PK * 2) + pn);
    if (next) {
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);   // MFMAs with weight 0
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // weight 0 refill
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // weight 1 refill
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The MFMA wavefronts' part of a job, for a wavefront holding NT token
// tiles of parity RH (NT = 0: it only takes the barriers).
template <bool GATEUP, int NT, int RH>
__device__ __forceinline__ void consume_job(int nK, int lane, int cq, int rows, int d, int f,
                                            const __bf16* lds, uint16_t* hdst, float* odst) {
  const __bf16* abuf = lds;
  const __bf16* bbuf = lds + A_BUFS * A_TILE;
  f32x16 acc[NT > 0 ? NT : 1][2];
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  step_barrier();   // step 0 is in buffers 0
  for (int ks = 0; ks < nK; ++ks) {
    if (NT > 0)
      mfma_step<NT>(acc, abuf + (ks % A_BUFS) * A_TILE, bbuf + (ks & 1) * B_TILE, lane, RH, cq);
    step_barrier();
  }
  if (NT == 0) return;

  // epilogue: lane l holds token 32(rh + 2i) + l%32; registers 4q..4q+3 of
  // tile j hold 4 consecutive columns.  The row stride and this lane's token
  // are hidden from the optimizer so that per-element offsets are not hoisted
  // out of the job loop.
  uint32_t ld = GATEUP ? f : d;
  int mt = 32 * RH + (lane & 31);
  opaque(ld);
  opaque(mt);
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int m = mt + 64 * i;
    if (m < rows) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (GATEUP) {
          uint2 v;
          v.x = pack_bf16x2(silu_fast(acc[i][0][4 * q]) * acc[i][1][4 * q],
                            silu_fast(acc[i][0][4 * q + 1]) * acc[i][1][4 * q + 1]);
          v.y = pack_bf16x2(silu_fast(acc[i][0][4 * q + 2]) * acc[i][1][4 * q + 2],
                            silu_fast(acc[i][0][4 * q + 3]) * acc[i][1][4 * q + 3]);
          *reinterpret_cast<uint2*>(hdst + static_cast<uint32_t>(m) * ld + 8 * q) = v;
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                         acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
            *reinterpret_cast<float4*>(odst + static_cast<uint32_t>(m) * ld + 32 * j + 8 * q) = v;
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// GATEUP: A = gathered x rows (bf16 [T][d]), B = G rows, epilogue silu(g)*u -> H bf16.
// !GATEUP: A = H rows of the group, B = D rows, epilogue fp32 rows.
// Wavefronts 0..7 run the MFMAs, 8..11 load and dequantize; both walk the
// same jobs and take the same barriers.
template <int FMT, bool GATEUP>
__global__ __launch_bounds__(PTHREADS) void prefill_gemm_kernel(
    const uint8_t* __restrict__ pool, int64_t slot_bytes, Planes P, int d, int f, GroupInfo g,
    const uint16_t* __restrict__ a_src, uint16_t* __restrict__ h_out,
    float* __restrict__ out_pairs, float* __restrict__ out_shared) {
  extern __shared__ __attribute__((aligned(16))) __bf16 lds[];
  const int K = GATEUP ? d : f;              // reduction length
  const int N = GATEUP ? 2 * f : d;          // output columns of the job space
  const int nK = K / PK;
  const int n_slices = (N + PN - 1) / PN;
  const int n_gm = g.tile_base[g.E + 1];     // (group, 256-row chunk) items
  const int total = ((n_gm + 7) / 8) * 8 * n_slices;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (wave < NCONS / 64) {
    const int lane = tid & 63;
    // wavefronts w and w + 4 share a SIMD: they take the two token-tile
    // parities of the same columns, so every SIMD gets half of the rows
    const int cq = wave & 3;                 // columns 64cq .. 64cq + 63
    const int rh = wave >> 2;                // token tiles rh, rh + 2, rh + 4, rh + 6
    for (int job = blockIdx.x; job < total; job += gridDim.x) {
      // (the MFMA wavefronts' own lookup is hidden behind the producers'
      // first loads of the job)
      int ns = 0;
      TileInfo ti;
      if (!fetch_job(g, n_slices, n_gm, total, job, ns, ti)) continue;   // uniform
      const int rows = ti.rows;
      const int row_tiles = (rows + 31) >> 5;
      const bool cols_ok = GATEUP ? (ns * (PN / 2) + 32 * cq < f) : (ns * PN + 64 * cq < d);
      const int nt = cols_ok ? min(4, max(0, (row_tiles - rh + 1) >> 1)) : 0;
      uint16_t* hdst = nullptr;
      float* odst = nullptr;
      if (GATEUP) {
        hdst = h_out + static_cast<int64_t>(ti.row_base + ti.m0) * f + ns * (PN / 2) + 32 * cq +
               4 * (lane >> 5);
      } else {
        odst = (ti.group < g.E ? out_pairs + static_cast<int64_t>(ti.row_base + ti.m0) * d
                               : out_shared + static_cast<int64_t>(ti.m0) * d) +
               static_cast<int64_t>(ns) * PN + 64 * cq + 4 * (lane >> 5);
      }
#define BITFFN_CONSUME(NT_, RH_) \
  consume_job<GATEUP, NT_, RH_>(nK, lane, cq, rows, d, f, lds, hdst, odst)
      switch (2 * nt + rh) {   // uniform per wavefront
        case 8: BITFFN_CONSUME(4, 0); break;
        case 9: BITFFN_CONSUME(4, 1); break;
        case 6: BITFFN_CONSUME(3, 0); break;
        case 7: BITFFN_CONSUME(3, 1); break;
        case 4: BITFFN_CONSUME(2, 0); break;
        case 5: BITFFN_CONSUME(2, 1); break;
        case 2: BITFFN_CONSUME(1, 0); break;
        case 3: BITFFN_CONSUME(1, 1); break;
        default: BITFFN_CONSUME(0, 0); break;
      }
#undef BITFFN_CONSUME
    }
  } else {
    ProdCtx c;
    c.p = tid - NCONS;
    c.nK = nK;
    // x is [T][d]; H is [T*k + T][f], under 4 GiB (checked by the entry point)
    c.a_rs = buf_rsrc(a_src, GATEUP ? static_cast<uint32_t>(g.T) * d * 2
                                    : static_cast<uint32_t>(g.T * (g.k + 1)) * f * 2);
    const int lane = c.p & 63, pw = c.p >> 6;
    // the next job's tile is fetched while the current one runs
    int ns_n = 0;
    TileInfo ti_n = {};
    bool ok_n = fetch_job(g, n_slices, n_gm, total, blockIdx.x, ns_n, ti_n);
    for (int job = blockIdx.x; job < total; job += gridDim.x) {
      const int ns = ns_n;
      const TileInfo ti = ti_n;
      const bool ok = ok_n;
      ok_n = fetch_job(g, n_slices, n_gm, total, job + gridDim.x, ns_n, ti_n);
      if (!ok) continue;                     // uniform
      c.b_rs = buf_rsrc(pool + static_cast<int64_t>(ti.slot) * slot_bytes,
                        static_cast<uint32_t>(slot_bytes));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ar0 = 64 * pw + 8 * j + (lane >> 3);
        const int ar = min(ar0, ti.rows - 1);
        const uint32_t row = GATEUP ? static_cast<uint32_t>(tile_token(g, ti, ti.m0 + ar))
                                    : static_cast<uint32_t>(ti.row_base + ti.m0 + ar);
        c.a_voff[j] = ar0 < ti.rows ? row * (2u * K) + 16u * ((lane & 7) ^ swz(ar0 & 15))
                                    : 0xFFFFFF00u;
      }
      if (GATEUP) {   // weight rows: tile 2j = gate, tile 2j+1 = up of h block j
        const int h = min(ns * (PN / 2) + (c.p >> 6) * 32 + (c.p & 31), f - 1);
        const uint32_t b_row = 2u * h + ((c.p >> 5) & 1);
        c.vb[0] = 2u * b_row;
        c.vb[1] = 2u * b_row + 1u;
      } else {
        const uint32_t b_row = min(ns * PN + c.p, d - 1);
        c.vb[0] = b_row;
        c.vb[1] = static_cast<uint32_t>(d) + b_row;
      }
      produce_job<FMT, GATEUP>(c, P, d, f, lds, lds + A_BUFS * A_TILE);
    }
  }
}

struct PrefillWs {
  GroupWorkspace gws;
  int32_t* perm;
  int32_t* tile_base;
  int32_t* tile_group;
  int32_t* group_slot;
  uint16_t* h;
};

// upper bound on (group, 256-row chunk) tiles: every group rounds up once,
// plus the shared expert's group of T rows
int64_t max_tiles(int T, int k, int E) {
  return (static_cast<int64_t>(T) * k + PM - 1) / PM + E + (T + PM - 1) / PM;
}

PrefillWs prefill_ws(void* ws, int d, int f, int T, int k, int E) {
  (void)d;
  (void)f;
  char* p = static_cast<char*>(ws);
  PrefillWs w;
  w.gws = group_workspace(p, T, E);
  p += group_workspace_bytes(T, E);
  w.perm = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<int64_t>(T) * k * 4);
  w.tile_base = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<int64_t>(E + 2) * 4);
  w.tile_group = reinterpret_cast<int32_t*>(p);
  p += align256(max_tiles(T, k, E) * 4);
  w.group_slot = reinterpret_cast<int32_t*>(p);
  p += align256(static_cast<int64_t>(E) * 4);
  w.h = reinterpret_cast<uint16_t*>(p);
  return w;
}

// Persistent grid: one workgroup per CU, a multiple of 8 so that job j and
// workgroup j mod grid share an XCD.
int prefill_grid(int64_t max_jobs) {
  const int n_cu = device_cus();
  int64_t grid = (max_jobs + 7) / 8 * 8;
  const int64_t cap = (n_cu + 7) / 8 * 8;
  if (grid > cap) grid = cap;
  return static_cast<int>(grid > 8 ? grid : 8);
}

template <int FMT, bool GATEUP>
hipError_t launch_gemm(const GroupInfo& g, int64_t max_jobs, const moe_layer& L, Planes P,
                       const uint16_t* a, uint16_t* h, float* out_pairs, float* out_shared,
                       hipStream_t s) {
  // the dynamic LDS limit is raised once per instantiation and device
  // (devices beyond the table every time)
  static std::atomic<uint64_t> lds_set{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < kMaxDevices ? uint64_t{1} << dev : 0;
  if (bit == 0 || !(lds_set.load(std::memory_order_relaxed) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_gemm_kernel<FMT, GATEUP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(PREFILL_LDS));
    if (e != hipSuccess) return e;
    lds_set.fetch_or(bit, std::memory_order_relaxed);
  }
  prefill_gemm_kernel<FMT, GATEUP><<<prefill_grid(max_jobs), PTHREADS, PREFILL_LDS, s>>>(
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
  g.tile_group = w.tile_group;
  g.group_slot = w.group_slot;
  g.E = L.n_experts;
  g.T = T;
  g.k = L.top_k;
  g.shared_slot = out_shared ? L.shared_slot : -1;
  (void)slot;
  const int64_t max_gm = max_tiles(T, L.top_k, L.n_experts);
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
         static_cast<size_t>(align256(max_tiles(T, k, E) * 4)) +
         static_cast<size_t>(align256(static_cast<int64_t>(E) * 4)) +
         static_cast<size_t>(align256((static_cast<int64_t>(T) * k + T) * f * 2));
}

hipError_t launch_prefill(const moe_layer& L, const uint16_t* x_bf16, int T, const int32_t* idx,
                          const int32_t* slot, float* out_pairs, int32_t* pair_pos,
                          int32_t* expert_offsets, float* out_shared, void* ws, hipStream_t s) {
  const PrefillWs w = prefill_ws(ws, L.d_model, L.d_ff, T, L.top_k, L.n_experts);
  // the pairs whose slot lies in the pool; the others are misses
  hipError_t e = launch_group_pairs(idx, slot, nullptr, T, L.top_k, L.n_experts, true,
                                    L.n_slots, w.gws,
                                    expert_offsets, w.perm, pair_pos, nullptr, nullptr,
                                    w.tile_base, PM, w.tile_group, w.group_slot, s);
  if (e != hipSuccess) return e;
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
