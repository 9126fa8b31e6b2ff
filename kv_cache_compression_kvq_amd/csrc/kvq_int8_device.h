// Per-row symmetric INT8 encoding, shared by every kernel that writes codes
// (symmetric INT8 formula of the Q-TensorFormer model card, section 6:
// scale = max|x| / 127, code = nearest integer of x / scale in [-128, 127]).
#pragma once

#include "kvq_device.h"

namespace kvq {

// Scale from the row's max |x| (bit pattern of a non-negative float); IEEE
// binary32 division.
__device__ __forceinline__ float row_scale(uint32_t amax_bits) {
  return __builtin_bit_cast(float, amax_bits) / 127.0f;
}

// Row divisor: the scale, or 1 for a zero scale (every value of such a row
// has |x| < 127 * 2^-150 and maps to code 0).
__device__ __forceinline__ float row_divisor(float s) { return (s == 0.0f) ? 1.0f : s; }

// One code: rint(RN32(x / s)) clamped to [-128, 127].  x / s is the
// compiler's IEEE binary32 division; rint rounds half to even.
__device__ __forceinline__ uint32_t code_of(float x, float sdiv) {
  const float t = x / sdiv;
  const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(t), -128.0f, 127.0f);
  return (uint32_t)(int)r & 0xFFu;
}

}  // namespace kvq
