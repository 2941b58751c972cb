// Device helpers shared by the kernels that write cache blocks (append and
// compaction): element offsets inside a (page, head) block, and the exact
// fp32 -> OCP e4m3 rounding.  The layout is the one pa.h documents.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

#pragma clang fp contract(off)

// Element offset of K(t, d) inside a (page, head) block: 64-byte column
// segments of 4*CE elements, CE = elements per 16-byte chunk.
template <int D, int E>
__device__ __forceinline__ int k_elem(int t, int d) {
  constexpr int SEG = 64 / E;
  return (d / SEG) * (kPageSize * SEG) + t * SEG + (d % SEG);
}

// Element offset of V(t, d): transposed, token-minor 16 x 4 tiles, grouped so
// that each 16-byte chunk holds TPC tiles of 4 tokens for one dim column.
template <int D, int E>
__device__ __forceinline__ int v_elem(int t, int d) {
  constexpr int TPC = 4 / E;
  const int c = d & 15, j = d >> 4;
  return ((((j / TPC) * 16 + c) * 4 + (t >> 2)) * TPC + (j % TPC)) * 4 + (t & 3);
}

// fp32 -> e4m3 code: saturate magnitudes above 448, round to nearest even on
// the integer bits, keep the sign of values that round to zero, NaN -> 0x7F.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;
  if (a > 0x43E00000u) a = 0x43E00000u;          // 448.0f
  uint32_t mag;
  if (a < 0x3C800000u) {                          // below 2^-6: subnormal grid of 2^-9
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // exact scaling, RNE
  } else {
    const uint32_t e = (a >> 23) - 120u;          // unbiased + 7
    const uint32_t keep = (a >> 20) & 7u;
    const uint32_t rest = a & 0xFFFFFu;
    const uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
    mag = ((e << 3) | keep) + up;                 // a mantissa carry bumps the exponent
  }
  return sign | mag;
}

__device__ __forceinline__ float bf16_value(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

}  // namespace pa
