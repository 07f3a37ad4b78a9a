// Device-side helpers shared by the attention kernels (gfx950 / CDNA4).
//
// Register layouts used throughout (wave64, v_mfma_f32_32x32x16_bf16):
//   A operand  (32 x 16, row-major in the math): lane l holds row l % 32,
//              k = 8 * (l / 32) + 0..7 as 8 consecutive bf16.
//   B operand  (16 x 32): lane l holds column l % 32, k = 8 * (l / 32) + 0..7.
//   C/D        (32 x 32 fp32): lane l, register r holds row
//              8 * (r / 4) + 4 * (l / 32) + (r % 4), column l % 32.
// A product whose output feeds the next product as an operand therefore keeps
// the "column" dimension in the lane index; the kernels arrange their
// products so each lane owns one query (forward) or one key (backward).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Both halves of the wave exchange values with the lane 32 away and return
// the pair (own, partner) in some order; callers only combine symmetrically.
__device__ __forceinline__ float max_with_lane_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_with_lane_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// fp32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Low halves of a and b as one word (a in the low 16 bits).
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
// High halves of a and b as one word (a's high half in the low 16 bits).
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace fa
