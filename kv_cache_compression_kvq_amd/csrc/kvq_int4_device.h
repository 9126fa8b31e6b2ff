// Asymmetric group-wise INT4 encoding, shared by every kernel that writes
// INT4 codes (asymmetric group-wise INT4 formula of the Q-TensorFormer model
// card, section 6: step = (max - min) / 15, offset = min, code = nearest
// integer of (x - offset) / step in [0, 15], reconstruction code * step +
// offset).
#pragma once

#include "kvq_device.h"

namespace kvq {

// Min over aligned segments of SEG lanes; every lane of a segment receives
// the segment's min.  All 64 lanes must be active.
template <int SEG>
__device__ __forceinline__ float seg_min_f32(float v) {
  if constexpr (SEG >= 2) v = __builtin_fminf(v, dpp_f32<kDppXor1>(v));
  if constexpr (SEG >= 4) v = __builtin_fminf(v, dpp_f32<kDppXor2>(v));
  if constexpr (SEG >= 8) v = __builtin_fminf(v, dpp_f32<kDppHalfMirror>(v));
  if constexpr (SEG >= 16) v = __builtin_fminf(v, dpp_f32<kDppMirror>(v));
  if constexpr (SEG >= 32) v = __builtin_fminf(v, swz_xor16_f32(v));
  if constexpr (SEG >= 64) v = __builtin_fminf(v, xor32_f32(v));
  return v;
}

// Step from the group's min and max (IEEE binary32 subtraction and
// division), and the divisor used for the codes: 1 for a zero step (every
// x - z of such a group is below 15 * 2^-150, so its code is 0).
__device__ __forceinline__ float group_step(float mn, float mx) { return (mx - mn) / 15.0f; }
__device__ __forceinline__ float step_divisor(float s) { return (s == 0.0f) ? 1.0f : s; }

// One code by division: rint(RN32(RN32(x - z) / sdiv)) in [0, 15].
__device__ __forceinline__ uint32_t nibble_of(float x, float z, float sdiv) {
  const float t = (x - z) / sdiv;
  return (uint32_t)(int)__builtin_amdgcn_fmed3f(__builtin_rintf(t), 0.0f, 15.0f);
}

// Whether q = t * rcp(s) may stand in for RN32(t / s): s in [2^-120, 2^120].
__device__ __forceinline__ bool rcp_ok(float sdiv) {
  return sdiv >= 0x1p-120f && sdiv <= 0x1p120f;
}

// Codes of N values of one group, as floats in [0, 15]: the codes of the
// division with one multiply per value.  For s in [2^-120, 2^120],
// v_rcp_f32 is within 1 ulp, so q = RN32(t * r) differs from RN32(t / s) by
// at most 15 * (2^-23 + 2^-24) + 2^-21 < 3.3e-6 (t / s <= 15 + 2^-19): both
// round to the same integer unless q lies within 2^-16 of a half-integer.
// Lanes with such a q (or a step outside the range) divide.
template <int N>
__device__ __forceinline__ void codes_rcp(const float (&x)[N], float z, float sdiv, float r,
                                          bool divide, float (&c)[N]) {
  float t[N];
  bool near = divide;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    t[e] = x[e] - z;
    const float q = t[e] * r;
    c[e] = __builtin_rintf(q);
    near |= __builtin_fabsf(q - c[e]) > 0.5f - 0x1p-16f;
  }
  if (near) {
    // (an opaque statement keeps the divisions behind the branch instead of
    // being computed for every lane and selected)
    __asm__ volatile("");
#pragma unroll
    for (int e = 0; e < N; ++e) c[e] = __builtin_rintf(t[e] / sdiv);
  }
#pragma unroll
  for (int e = 0; e < N; ++e) c[e] = __builtin_amdgcn_fmed3f(c[e], 0.0f, 15.0f);
}

// N codes (floats in [0, 15]) packed four bits each, element e at bit 4e.
template <int N>
__device__ __forceinline__ uint32_t pack_nibbles(const float (&c)[N]) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) w |= (uint32_t)(int)c[e] << (4 * e);
  return w;
}

// RN32(RN32(c * s) + z), kept as two roundings.
__device__ __forceinline__ float recon4(float c, float s, float z) {
#pragma clang fp contract(off)
  return c * s + z;
}

}  // namespace kvq
