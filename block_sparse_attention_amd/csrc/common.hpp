// Device-side helpers shared by the bsattn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsattn {

constexpr int kBlock = 64;     // tokens per query block and per key/value block
constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define BSATTN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bfloat16 (round to nearest even) in one dword, lo in bits 0..15.
// Lowered to a single v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of a lane's value and the value held by lane ^ 32.
__device__ __forceinline__ float max_with_half_swap(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return fmaxf(__int_as_float(s[0]), __int_as_float(s[1]));
}
__device__ __forceinline__ float sum_with_half_swap(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(s[0]) + __int_as_float(s[1]);
}

__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace bsattn
