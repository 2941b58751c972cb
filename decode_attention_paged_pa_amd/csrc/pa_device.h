// Device helpers for the gfx950 kernels: vector types, exact FP8 decoding,
// BF16 rounding and cross-lane reductions of a 64-lane wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> BF16 bits, round to nearest even (NaN -> quiet NaN).
__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Four e4m3 codes (one dword, byte i = element i) -> four BF16 values packed in
// two dwords.  The hardware conversion to fp32 is exact for OCP e4m3 on gfx950,
// and every e4m3 value fits in BF16's 8-bit significand, so keeping the upper
// half of each fp32 is exact as well.
__device__ inline u32x2 fp8x4_to_bf16x4(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  u32x2 r;
  r.x = __builtin_amdgcn_perm(__float_as_uint(lo.y), __float_as_uint(lo.x), 0x07060302u);
  r.y = __builtin_amdgcn_perm(__float_as_uint(hi.y), __float_as_uint(hi.x), 0x07060302u);
  return r;
}

// Four e4m3 codes -> four f16 values (exact: e4m3's range and precision are
// inside f16's, subnormals included).
__device__ inline f16x4 fp8x4_to_f16x4(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  auto a = __builtin_amdgcn_cvt_pkrtz(lo.x, lo.y);
  auto b = __builtin_amdgcn_cvt_pkrtz(hi.x, hi.y);
  f16x4 r;
  r[0] = (_Float16)a[0];
  r[1] = (_Float16)a[1];
  r[2] = (_Float16)b[0];
  r[3] = (_Float16)b[1];
  return r;
}

// Reductions over the four lanes {l, l^16, l^32, l^48} (one MFMA column).
// permlane32_swap(x, x) yields {x[l & 31], x[(l & 31) + 32]} and
// permlane16_swap(x, x) yields {x[l & ~16], x[l | 16]}: both lanes of a pair
// combine the same two values, so all four lanes end with the same result.
__device__ inline float col_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ inline float col_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

}  // namespace pa
