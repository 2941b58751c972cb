// Device helpers for the gfx950 kernels: vector types, exact FP8 decoding,
// BF16 rounding and cross-lane reductions of a 64-lane wavefront.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
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

// Four e4m3 codes (one dword, byte i = element i) -> four BF16 / f16 values
// packed in two dwords; every e4m3 value is exactly representable in both.
#ifndef PA_SCALED_CVT
#define PA_SCALED_CVT 1
#endif
#if PA_SCALED_CVT
// gfx950's scaled pair conversions decode two codes per instruction; with a
// scale of 1.0 they are exact (checked against the OCP definition for all 256
// codes).  The packed result is only ever used as a whole dword: extracting
// single halves from these builtins' results has produced wrong code.
// Measured on MI355X: the same as the two-step conversion where the kernels
// stream memory, 7% faster for the 8-draft FP8 kernel (bit-identical outputs).
__device__ inline u32x2 fp8x4_to_bf16x4(uint32_t w) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}

__device__ inline u32x2 fp8x4_to_f16x4(uint32_t w) {
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
  return r;
}
#else
// The conversion to fp32 is exact for OCP e4m3 on gfx950 (checked for all 256
// codes); keeping the upper half of each fp32 is then an exact BF16, and the
// round-toward-zero pack to f16 is exact too.
__device__ inline u32x2 fp8x4_to_bf16x4(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  u32x2 r;
  r.x = __builtin_amdgcn_perm(__float_as_uint(lo.y), __float_as_uint(lo.x), 0x07060302u);
  r.y = __builtin_amdgcn_perm(__float_as_uint(hi.y), __float_as_uint(hi.x), 0x07060302u);
  return r;
}

__device__ inline u32x2 fp8x4_to_f16x4(uint32_t w) {
  f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo.x, lo.y));
  r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(hi.x, hi.y));
  return r;
}
#endif

// Exact decode of one e4m3 code (byte 0 of `code`) to fp32.
__device__ inline float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(code, false)[0];
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

// The 32x32x16 MFMA operand (8 halves of one row or column: k = 8 (l >> 5) ..
// + 7) from the 16x16x16 operands of two tiles a and b (4 halves each: lane
// (c, q) holds k = 4 q .. 4 q + 3 of row or column c).  v_permlane16_swap
// exchanges the odd 16-lane rows of its first operand with the even rows of
// its second, so per dword the first result holds rows {a0, b0, a2, b2} and
// the second {a1, b1, a3, b3}: lane l then holds k 0-7 (l < 32) or 8-15 of
// row (or column) l & 31 -- a's rows for l & 16 clear, b's for it set.
__device__ inline u32x4 pair_rows(u32x2 a, u32x2 b) {
  auto s0 = __builtin_amdgcn_permlane16_swap(a.x, b.x, false, false);
  auto s1 = __builtin_amdgcn_permlane16_swap(a.y, b.y, false, false);
  return u32x4{s0[0], s1[0], s0[1], s1[1]};
}

// a in lanes whose bit 4 is clear, b in the others (lanes 16-31 and 48-63:
// the second column tile of a 32-column pair).  Written as one v_cndmask with
// a constant lane mask: as a C++ select between two array elements the
// compiler turned it into a lane-indexed stack array, whose reload waited
// for every outstanding memory load.
__device__ inline float pick_hi16(float a, float b) {
  float r;
  asm("v_cndmask_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(0xFFFF0000FFFF0000ull));
  return r;
}

// Maximum over the 64 lanes of a wave (NaN inputs are ignored by fmaxf).
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int d = 32; d > 0; d >>= 1) x = fmaxf(x, __shfl_xor(x, d, 64));
  return x;
}

__device__ inline float col_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

}  // namespace pa
