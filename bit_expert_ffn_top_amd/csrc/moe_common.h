// Shared definitions for the gfx950 kernels of the routed-expert MoE layer.
//
// Slot layout (one packed expert): matrix G (2*d_ff x d_model, gate row j at
// 2j, up row j at 2j+1) then D (d_model x d_ff).  Each matrix is row-major in
// 32-weight blocks stored as planes (codes, [hi], scale, [min]), every plane
// starting 256-byte aligned from the slot start.
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

// Sum over the 32 weights of one block of w_j * x_j where w_j decodes from
// `lo` (2-bit codes, LSB first, 16 per word) and, for Q3G, `hi` (bit j = bit
// 2 of code j).  `xs` = sum of the 32 x_j.
template <int FMT>
__device__ __forceinline__ float block_dot(uint32_t lo0, uint32_t lo1, uint32_t hi,
                                           float s, float m, const float* x, float xs) {
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t q = (lo0 >> (2 * j)) & 3u;
    if (FMT == MOE_FMT_Q3G) q |= ((hi >> j) & 1u) << 2;
    acc = fmaf(static_cast<float>(q), x[j], acc);
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t q = (lo1 >> (2 * j)) & 3u;
    if (FMT == MOE_FMT_Q3G) q |= ((hi >> (16 + j)) & 1u) << 2;
    acc = fmaf(static_cast<float>(q), x[16 + j], acc);
  }
  if (FMT == MOE_FMT_Q2S) return s * (acc - 1.5f * xs);
  if (FMT == MOE_FMT_Q2SM) return fmaf(s, acc, m * xs);
  // Q3G: w = s*(2q-7)/7  ->  sum = s*(2*acc/7 - xs)
  return s * fmaf(acc, 2.0f / 7.0f, -xs);
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
