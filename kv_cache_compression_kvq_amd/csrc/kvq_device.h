// Device-side helpers shared by the libkvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// --- cross-lane moves --------------------------------------------------------
// DPP controls (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i inside each 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i inside each 16

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Exchange with lane ^ 16 inside each 32-lane half (ds_swizzle bit mode:
// and_mask 0x1f, or_mask 0, xor_mask 0x10).
__device__ __forceinline__ uint32_t swz_xor16_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}
__device__ __forceinline__ float swz_xor16_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
}
// Exchange with lane ^ 32 (v_permlane32_swap-free form: ds_bpermute).
__device__ __forceinline__ uint32_t xor32_u32(uint32_t v) {
  const int lane = __lane_id();
  return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, (int)v);
}
__device__ __forceinline__ float xor32_f32(float v) {
  return __builtin_bit_cast(float, (int)xor32_u32(__builtin_bit_cast(uint32_t, v)));
}

// Both halves' values of a 64-lane register: lo = the value of lane l % 32,
// hi = that of lane 32 + l % 32, in every lane (v_permlane32_swap of the
// register with itself; no LDS traffic).
__device__ __forceinline__ void halves_u32(uint32_t v, uint32_t& lo, uint32_t& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = r[0];
  hi = r[1];
}

// Max over aligned segments of SEG lanes (power of two, <= 64); every lane
// of a segment receives the segment's max.  All 64 lanes must be active.
template <int SEG>
__device__ __forceinline__ uint32_t seg_max_u32(uint32_t v) {
  if constexpr (SEG >= 2) v = max(v, dpp_u32<kDppXor1>(v));
  if constexpr (SEG >= 4) v = max(v, dpp_u32<kDppXor2>(v));
  if constexpr (SEG >= 8) v = max(v, dpp_u32<kDppHalfMirror>(v));
  if constexpr (SEG >= 16) v = max(v, dpp_u32<kDppMirror>(v));
  if constexpr (SEG >= 32) v = max(v, swz_xor16_u32(v));
  if constexpr (SEG >= 64) v = max(v, xor32_u32(v));
  return v;
}

// Sum over aligned segments of SEG lanes; every lane receives the sum.
template <int SEG>
__device__ __forceinline__ float seg_sum_f32(float v) {
  if constexpr (SEG >= 2) v = v + dpp_f32<kDppXor1>(v);
  if constexpr (SEG >= 4) v = v + dpp_f32<kDppXor2>(v);
  if constexpr (SEG >= 8) v = v + dpp_f32<kDppHalfMirror>(v);
  if constexpr (SEG >= 16) v = v + dpp_f32<kDppMirror>(v);
  if constexpr (SEG >= 32) v = v + swz_xor16_f32(v);
  if constexpr (SEG >= 64) v = v + xor32_f32(v);
  return v;
}

template <int SEG>
__device__ __forceinline__ float seg_max_f32(float v) {
  if constexpr (SEG >= 2) v = __builtin_fmaxf(v, dpp_f32<kDppXor1>(v));
  if constexpr (SEG >= 4) v = __builtin_fmaxf(v, dpp_f32<kDppXor2>(v));
  if constexpr (SEG >= 8) v = __builtin_fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  if constexpr (SEG >= 16) v = __builtin_fmaxf(v, dpp_f32<kDppMirror>(v));
  if constexpr (SEG >= 32) v = __builtin_fmaxf(v, swz_xor16_f32(v));
  if constexpr (SEG >= 64) v = __builtin_fmaxf(v, xor32_f32(v));
  return v;
}

// --- streaming memory access ----------------------------------------------------
// Loads and stores of data touched once: nontemporal, so streams do not
// displace reused lines in L2 / MALL (measured on MI355X: a 16-byte-per-lane
// read stream reaches ~7.0 TB/s nontemporal vs ~6.25 TB/s with default
// caching).
template <typename V>
__device__ __forceinline__ V ld_stream(const V* p) {
  return __builtin_nontemporal_load(p);
}
template <typename V>
__device__ __forceinline__ void st_stream(V* p, const V& v) {
  __builtin_nontemporal_store(v, p);
}

// --- element access -----------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }

__device__ __forceinline__ uint32_t abs_bits(float v) {
  return __builtin_bit_cast(uint32_t, v) & 0x7FFFFFFFu;
}

// int8 lane k of a 32-bit word, converted exactly to float.
__device__ __forceinline__ float i8_to_f32(uint32_t w, int k) {
  return (float)(int8_t)(w >> (8 * k));
}

// Round-to-nearest-even binary32 -> binary16 bit pattern.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

}  // namespace kvq
