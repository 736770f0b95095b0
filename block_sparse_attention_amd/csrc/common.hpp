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

// Order key of column c with score x: a larger key is a larger score, and
// among equal scores the lower column; -0.0 and +0.0 are equal scores.  Every
// key of a column below 2^32 - 1 is nonzero.
__device__ __forceinline__ uint64_t rank_key(float x, int c) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) == 0) u = 0;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)c);
}

// The score and column a rank_key encodes (a zero score comes back as +0.0).
__device__ __forceinline__ float rank_key_score(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ int rank_key_column(uint64_t key) {
  return (int)(0xffffffffu - (uint32_t)key);
}

// Top-k cut over a wave by a bitwise radix select.  key[u] holds the order
// key of column 64 u + lane (distinct keys; 0 for padding, below every real
// key); chunks u >= nch are not read.  On return the selected columns are
// exactly those with (key & hm) >= prefix: walking the key bits from the top,
// the prefix of the topk-th largest key is fixed one bit at a time from
// ballot counts, stopping as soon as the keys on the prefix are exactly the
// ones still needed.  Requires 0 < topk < number of real keys.
template <int NCH>
__device__ __forceinline__ void wave_topk_cut(const uint64_t (&key)[NCH], int nch, int topk,
                                              uint64_t& hm, uint64_t& prefix) {
  int want = topk;
  prefix = 0;
  hm = 0;
  for (int bit = 63; bit >= 0; --bit) {
    const uint64_t m = ~0ull << bit;
    const uint64_t target = prefix | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < NCH; ++u)
      if (u < nch) cnt += __popcll(wave_ballot((key[u] & m) == target));
    int cand;
    if (cnt >= want) {
      prefix = target;
      cand = cnt;
    } else {
      want -= cnt;
      cand = 0;
#pragma unroll
      for (int u = 0; u < NCH; ++u)
        if (u < nch) cand += __popcll(wave_ballot((key[u] & m) == prefix));
    }
    hm = m;
    if (cand == want) break;
  }
}

// ---- wave-level memory and matrix-core primitives ----

// One wave-wide 16-byte-per-lane load straight into LDS: lane l reads
// base + voff_l (base uniform, voff a per-lane byte offset) and its 16 bytes
// go to LDS byte address lds + kLdsOff + 16 * l (M0 holds the uniform base).
template <uint32_t kLdsOff>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds), "i"(kLdsOff)
               : "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// The same, and every LDS operation of this wave has completed.
template <int N>
__device__ __forceinline__ void wait_vmem_lds0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier_raw() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x2 lds_read_tr16(uint32_t byte_addr) {
  bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((BSATTN_LDS bf16x4*)(uintptr_t)byte_addr);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x4 lds_read_b128(uint32_t byte_addr) {
  return *(const BSATTN_LDS u32x4*)(uintptr_t)byte_addr;
}

}  // namespace bsattn
