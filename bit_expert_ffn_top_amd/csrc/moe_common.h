// Shared definitions for the gfx950 kernels of the routed-expert MoE layer.
//
// Slot layout (one packed expert): matrix G (2*d_ff x d_model, gate row j at
// 2j, up row j at 2j+1) then D (d_model x d_ff), each cut into 32-weight
// blocks along its rows and stored unit-major: a unit is U consecutive blocks
// of one row (U = 2 for G, 1 for D), and unit c of row r (R rows) has index
// c*R + r, so one unit of consecutive rows is contiguous.  Each matrix is a
// sequence of planes (codes, [hi], scale, [min]) holding its units in index
// order, every plane starting 256-byte aligned from the slot start.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitffn_moe.h"

namespace bitffn {

struct Planes {
  int64_t codes, hi, scale, min;  // byte offsets from the slot start, -1 = absent
};

struct SlotLayout {
  Planes G, D;
  int64_t total;
};

__host__ __device__ inline int64_t align256(int64_t n) { return (n + 255) & ~int64_t(255); }

__host__ __device__ inline SlotLayout slot_layout(int fmt, int d, int f) {
  SlotLayout L;
  int64_t pos = 0;
  for (int m = 0; m < 2; ++m) {
    const int64_t rows = m == 0 ? 2 * int64_t(f) : int64_t(d);
    const int64_t cols = m == 0 ? int64_t(d) : int64_t(f);
    const int64_t nblk = rows * (cols / 32);
    Planes P{-1, -1, -1, -1};
    P.codes = pos;
    pos = align256(pos + nblk * 8);
    if (fmt == MOE_FMT_Q3G) {
      P.hi = pos;
      pos = align256(pos + nblk * 4);
    }
    P.scale = pos;
    pos = align256(pos + nblk * 2);
    if (fmt == MOE_FMT_Q2SM) {
      P.min = pos;
      pos = align256(pos + nblk * 2);
    }
    if (m == 0)
      L.G = P;
    else
      L.D = P;
  }
  L.total = pos;
  return L;
}

// ---------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// IEEE round-to-nearest-even of an fp32 value to bfloat16 bits (finite inputs).
__device__ __forceinline__ uint16_t float_to_bf16_rne(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}

// Makes `v` opaque to the optimizer at this point (no instruction is emitted),
// so work derived from it is not hoisted out of the enclosing loop.
template <typename T>
__device__ __forceinline__ void opaque(T& v) {
  static_assert(sizeof(T) % 4 == 0, "32-bit granules");
  uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
  for (unsigned i = 0; i < sizeof(T) / 4; ++i) asm volatile("" : "+v"(w[i]));
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// v + (v of another lane of the same row of 16 lanes), DPP control CTRL
template <int CTRL>
__device__ __forceinline__ float add_dpp_ctrl(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                 0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each row of 16 lanes, complete in every lane of the row (a fixed
// tree: pairs, quads, then rotations by 4 and 8).
__device__ __forceinline__ float row16_sum_dpp(float v) {
  v = add_dpp_ctrl<0xB1>(v);    // quad_perm [1,0,3,2]
  v = add_dpp_ctrl<0x4E>(v);    // quad_perm [2,3,0,1]
  v = add_dpp_ctrl<0x124>(v);   // row_ror:4
  return add_dpp_ctrl<0x128>(v);   // row_ror:8
}

// ---------------------------------------------------------------------------
// code extraction into fp16 pairs
//
// A 32-bit word of packed 2-bit codes (code i at bits [2i, 2i+2)) is turned
// into eight registers of two fp16 values each, value = c + q, by masking a
// (shifted) copy of the word and OR-ing a constant exponent: a code that sits
// at fp16 mantissa bits [p, p+2) under exponent 25 - p reads as 2^(10-p) + q.
// Code i is paired with code i + 8 (low and high half of one register).
// v_fma_mix_f32 then multiplies each half by an fp32 activation.  The offsets
// c (64, 16 or 4 by position) are removed once per block through the
// precomputed sum C = sum_j c_j x_j.
// ---------------------------------------------------------------------------

// (a & mask) | bits in one v_and_or_b32 (the two constants would otherwise
// cost a v_and and a v_or, since a VOP3 encoding takes no literal here).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(bits));
  return r;
}

__device__ __forceinline__ float h_lo(uint32_t r) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r)));
}
__device__ __forceinline__ float h_hi(uint32_t r) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(r >> 16)));
}

// offset c_j of position j (mod 16) for the 2-bit extraction below
__host__ __device__ constexpr float q2_offset(int j) {
  return (j % 8 == 2 || j % 8 == 5) ? 64.0f : (j % 8 == 0 || j % 8 == 3 || j % 8 == 6) ? 16.0f : 4.0f;
}
// offset c_j of position j for the 3-bit extraction below
__host__ __device__ constexpr float q3_offset(int j) { return (j % 2 == 0) ? 64.0f : 16.0f; }

// acc + sum_j (c_j + q_j) * x[j] over the 16 2-bit codes of `w`; two
// independent partial sums are carried in a0/a1.
template <typename XT>
__device__ __forceinline__ void dot16_q2(uint32_t w, const XT& x, int x0, float& a0, float& a1) {
  const uint32_t b = w >> 6, c = w << 6;
  const uint32_t r0 = and_or(w, 0x00300030u, 0x54005400u);  // 64+q2  | 64+q10
  const uint32_t r1 = and_or(w, 0x00C000C0u, 0x4C004C00u);  // 16+q3  | 16+q11
  const uint32_t r2 = and_or(w, 0x03000300u, 0x44004400u);  // 4+q4   | 4+q12
  const uint32_t r3 = and_or(b, 0x00300030u, 0x54005400u);  // 64+q5  | 64+q13
  const uint32_t r4 = and_or(b, 0x00C000C0u, 0x4C004C00u);  // 16+q6  | 16+q14
  const uint32_t r5 = and_or(b, 0x03000300u, 0x44004400u);  // 4+q7   | 4+q15
  const uint32_t r6 = and_or(c, 0x00C000C0u, 0x4C004C00u);  // 16+q0  | 16+q8
  const uint32_t r7 = and_or(c, 0x03000300u, 0x44004400u);  // 4+q1   | 4+q9
  a0 = fmaf(h_lo(r6), x[x0 + 0], a0);
  a1 = fmaf(h_lo(r7), x[x0 + 1], a1);
  a0 = fmaf(h_lo(r0), x[x0 + 2], a0);
  a1 = fmaf(h_lo(r1), x[x0 + 3], a1);
  a0 = fmaf(h_lo(r2), x[x0 + 4], a0);
  a1 = fmaf(h_lo(r3), x[x0 + 5], a1);
  a0 = fmaf(h_lo(r4), x[x0 + 6], a0);
  a1 = fmaf(h_lo(r5), x[x0 + 7], a1);
  a0 = fmaf(h_hi(r6), x[x0 + 8], a0);
  a1 = fmaf(h_hi(r7), x[x0 + 9], a1);
  a0 = fmaf(h_hi(r0), x[x0 + 10], a0);
  a1 = fmaf(h_hi(r1), x[x0 + 11], a1);
  a0 = fmaf(h_hi(r2), x[x0 + 12], a0);
  a1 = fmaf(h_hi(r3), x[x0 + 13], a1);
  a0 = fmaf(h_hi(r4), x[x0 + 14], a0);
  a1 = fmaf(h_hi(r5), x[x0 + 15], a1);
}

// Same for 16 3-bit codes: low bits in `w`, high bits in `hw` where the high
// bit of code i (i = 0..15 of this word) is at bit 2i + 1 + HOFF of `hw`
// (HOFF = 0 for codes 0..15 of a block, -1 for codes 16..31).  Each value is
// a 3-bit code at mantissa bits [p, p+3), p = 4 or 6: offset 64 or 16.
template <int HOFF, typename XT>
__device__ __forceinline__ void dot16_q3(uint32_t w, uint32_t hw, const XT& x, int x0, float& a0,
                                         float& a1) {
  const uint32_t wl = w << 4, wr4 = w >> 4, wr8 = w >> 8;
  const uint32_t h_m4 = HOFF == 0 ? (hw << 5) : (hw << 6);   // pairs (0,8),(1,9)
  const uint32_t h_0 = HOFF == 0 ? (hw << 1) : (hw << 2);    // pairs (2,10),(3,11)
  const uint32_t h_4 = HOFF == 0 ? (hw >> 3) : (hw >> 2);    // pairs (4,12),(5,13)
  const uint32_t h_8 = HOFF == 0 ? (hw >> 7) : (hw >> 6);    // pairs (6,14),(7,15)
  const uint32_t r0 = and_or(h_m4, 0x00400040u, and_or(wl, 0x00300030u, 0x54005400u));   // 0 | 8
  const uint32_t r1 = and_or(h_m4, 0x01000100u, and_or(wl, 0x00C000C0u, 0x4C004C00u));   // 1 | 9
  const uint32_t r2 = and_or(h_0, 0x00400040u, and_or(w, 0x00300030u, 0x54005400u));     // 2 | 10
  const uint32_t r3 = and_or(h_0, 0x01000100u, and_or(w, 0x00C000C0u, 0x4C004C00u));     // 3 | 11
  const uint32_t r4 = and_or(h_4, 0x00400040u, and_or(wr4, 0x00300030u, 0x54005400u));   // 4 | 12
  const uint32_t r5 = and_or(h_4, 0x01000100u, and_or(wr4, 0x00C000C0u, 0x4C004C00u));   // 5 | 13
  const uint32_t r6 = and_or(h_8, 0x00400040u, and_or(wr8, 0x00300030u, 0x54005400u));   // 6 | 14
  const uint32_t r7 = and_or(h_8, 0x01000100u, and_or(wr8, 0x00C000C0u, 0x4C004C00u));   // 7 | 15
  a0 = fmaf(h_lo(r0), x[x0 + 0], a0);
  a1 = fmaf(h_lo(r1), x[x0 + 1], a1);
  a0 = fmaf(h_lo(r2), x[x0 + 2], a0);
  a1 = fmaf(h_lo(r3), x[x0 + 3], a1);
  a0 = fmaf(h_lo(r4), x[x0 + 4], a0);
  a1 = fmaf(h_lo(r5), x[x0 + 5], a1);
  a0 = fmaf(h_lo(r6), x[x0 + 6], a0);
  a1 = fmaf(h_lo(r7), x[x0 + 7], a1);
  a0 = fmaf(h_hi(r0), x[x0 + 8], a0);
  a1 = fmaf(h_hi(r1), x[x0 + 9], a1);
  a0 = fmaf(h_hi(r2), x[x0 + 10], a0);
  a1 = fmaf(h_hi(r3), x[x0 + 11], a1);
  a0 = fmaf(h_hi(r4), x[x0 + 12], a0);
  a1 = fmaf(h_hi(r5), x[x0 + 13], a1);
  a0 = fmaf(h_hi(r6), x[x0 + 14], a0);
  a1 = fmaf(h_hi(r7), x[x0 + 15], a1);
}

// Per-block sums an activation vector needs: X = sum_j x_j and the offset sum
// C = sum_j c_j x_j of the format's extraction, folded into one constant K:
//   Q2S : block = s * (acc - K),               K = C + 1.5 X
//   Q2SM: block = s * (acc - K) + m * X,       K = C
//   Q3G : block = s * (acc * 2/7 - K),         K = C * 2/7 + X
template <int FMT>
__device__ __forceinline__ float block_offset_weight(int j) {
  return FMT == MOE_FMT_Q3G ? q3_offset(j) : q2_offset(j % 16);
}

template <int FMT>
__device__ __forceinline__ float block_const(float X, float C) {
  if (FMT == MOE_FMT_Q2S) return fmaf(1.5f, X, C);
  if (FMT == MOE_FMT_Q2SM) return C;
  return fmaf(C, 2.0f / 7.0f, X);
}

// One block's contribution added to `row`: s, m fp16 bits (low 16 bits used).
template <int FMT>
__device__ __forceinline__ float block_finish(float row, float acc, float K, float X, uint32_t s16,
                                              uint32_t m16) {
  const float s = half_bits_to_float(s16 & 0xFFFFu);
  if (FMT == MOE_FMT_Q2S) return fmaf(s, acc - K, row);
  if (FMT == MOE_FMT_Q2SM) return fmaf(half_bits_to_float(m16 & 0xFFFFu), X, fmaf(s, acc - K, row));
  return fmaf(s, fmaf(acc, 2.0f / 7.0f, -K), row);
}

// Dot of one 32-weight block with x[x0 .. x0+31]: `lo0`/`lo1` codes of
// positions 0-15 / 16-31, `hi` the block's high-bit word (3-bit format).
template <int FMT, typename XT>
__device__ __forceinline__ float block_acc(uint32_t lo0, uint32_t lo1, uint32_t hi, const XT& x,
                                           int x0) {
  float a0 = 0.0f, a1 = 0.0f;
  if (FMT == MOE_FMT_Q3G) {
    dot16_q3<0>(lo0, hi, x, x0, a0, a1);
    dot16_q3<-1>(lo1, hi, x, x0 + 16, a0, a1);
  } else {
    dot16_q2(lo0, x, x0, a0, a1);
    dot16_q2(lo1, x, x0 + 16, a0, a1);
  }
  return a0 + a1;
}

// Dequantized value of code q (Q3G: 3-bit) with fp32 scale s and min m, as the
// fp32 value nearest the exact one: s*(q-1.5) and s*q are exact, m + s*q is
// one rounding of an exact sum, and s*(2q-7) is exact before the single,
// correctly rounded division by 7.  Rounding that to bf16 then equals
// rounding the exact value (a quotient by 7 never lands on a bf16 tie).
template <int FMT>
__device__ __forceinline__ float dequant_one(uint32_t q, float s, float m) {
  if (FMT == MOE_FMT_Q2S) return s * (static_cast<float>(q) - 1.5f);
  if (FMT == MOE_FMT_Q2SM) return fmaf(s, static_cast<float>(q), m);
  return (s * static_cast<float>(2 * static_cast<int>(q) - 7)) / 7.0f;
}

}  // namespace bitffn
