// Loads for the QJL score kernels: sign words as whole 128-byte lines
// (with the lane exchange that gives every lane its token's words in the
// order the rotated lookups take), and the query projection with its query
// values read straight from memory.
#pragma once

#include "kvq_qjl_device.h"

namespace kvq {

// The same y = S q as project16_lite (bit for bit) when the workgroup's
// waves hold 4 RG rows each and together all m rows (m = 4 RG x waves), with
// the lane's 8 query values read straight from memory (no LDS staging, no
// workgroup barrier): issue() requests the rows and the query, wait() makes
// the wave wait for them, finish() writes the wave's rows of y (callers
// synchronise before reading y).
template <typename TQ, int RG>
struct QueryProjDirect {
  f16x8 raw[RG];
  TQ qraw[8];

  __device__ __forceinline__ void issue(const _Float16* __restrict__ S, const TQ* __restrict__ q,
                                        int d) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cc = min(lane & 15, d / 8 - 1);
#pragma unroll
    for (int it = 0; it < RG; ++it)
      raw[it] = *reinterpret_cast<const f16x8*>(
          S + (int64_t)(wave * 4 * RG + 4 * it + (lane >> 4)) * d + 8 * cc);
#pragma unroll
    for (int e = 0; e < 8; ++e) qraw[e] = q[8 * cc + e];
  }

  __device__ __forceinline__ void wait() {
#pragma unroll
    for (int it = 0; it < RG; ++it) asm volatile("" ::"v"(raw[it]));
#pragma unroll
    for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(qraw[e]));
  }

  __device__ __forceinline__ void finish(float* y, int d) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const bool live_c = 8 * c < d;
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = to_f32(qraw[e]);
#pragma unroll
    for (int it = 0; it < RG; ++it) {
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)raw[it][e], qv[e], part);
      part = seg_sum_f32<16>(live_c ? part : 0.0f);
      if (c == 0) y[wave * 4 * RG + 4 * it + (lane >> 4)] = part;
    }
  }
};

// Sign words of a wave's tokens, read as whole 128-byte lines.
//
// The lookups want, in lane L, the 8 words of the lane's token with the two
// 16-byte halves ordered by bit 4 of r = L mod 32: words 0..3 are half
// h = (r >> 4) & 1, words 4..7 half h ^ 1 (the first step of the rotation by
// r bytes).  Loading those halves lane by lane (load_rot_words) makes every
// wave instruction touch 64 lines and use half of each, which streams from
// HBM well below the rate of whole lines when the sign words are most of
// the bytes, as in the score kernels.  (The decode kernels keep
// load_rot_words: there the value codes dominate the bytes, and the lane
// exchange costs more than whole lines gain.)  Here every load instruction reads 32 consecutive
// tokens (1 KiB): lanes L and L + 32 read the two halves of one token, each
// the half its own rotation starts with, and v_permlane32_swap (exchange of
// the upper 32 lanes of one register with the lower 32 of another) moves the
// other half across.  The words that reach each lane are the same either
// way, so the scores do not change.  All 64 lanes must execute the swaps.
//
// Tokens past t_last re-read token t_last (their lanes store nothing).

// 64 tokens t_first .. t_first + 63, lane L scoring token t_first + L: x
// holds the halves of tokens t_first + L mod 32, y those of t_first + 32 +
// L mod 32.  blk: sign words of token 0 of the range.
struct RotWords64 {
  u32x4 x, y;
};
// (Offsets are unsigned 32-bit bytes from the uniform base, which the
// loads take as a scalar base plus a 32-bit lane offset.)
__device__ __forceinline__ const u32x4* rot_half_ptr(const uint32_t* blk, int t, int hsel) {
  return reinterpret_cast<const u32x4*>(reinterpret_cast<const unsigned char*>(blk) +
                                        ((uint32_t)t * 32u + 16u * (uint32_t)hsel));
}
__device__ __forceinline__ void issue_rot_words64(const uint32_t* blk, int t_first, int t_last,
                                                  int lane, RotWords64& rw) {
  const int hsel = ((lane >> 4) & 1) ^ (lane >> 5);
  rw.x = ld_stream(rot_half_ptr(blk, min(t_first + (lane & 31), t_last), hsel));
  rw.y = ld_stream(rot_half_ptr(blk, min(t_first + 32 + (lane & 31), t_last), hsel));
}
// Lower lanes keep x (their first half) and receive the upper lanes' x (the
// second); upper lanes receive the lower lanes' y (their first) and keep y.
__device__ __forceinline__ void finish_rot_words64(const RotWords64& rw, uint32_t w[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto sw = __builtin_amdgcn_permlane32_swap(rw.x[k], rw.y[k], false, false);
    w[k] = sw[0];
    w[4 + k] = sw[1];
  }
}

// 32 tokens t_first .. t_first + 31, lanes L and L + 32 both scoring token
// t_first + L mod 32 (for different queries): one instruction.
__device__ __forceinline__ u32x4 issue_rot_words32(const uint32_t* blk, int t_first, int t_last,
                                                   int lane) {
  const int hsel = ((lane >> 4) & 1) ^ (lane >> 5);
  return ld_stream(rot_half_ptr(blk, min(t_first + (lane & 31), t_last), hsel));
}
__device__ __forceinline__ void finish_rot_words32(u32x4 x, uint32_t w[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const auto sw = __builtin_amdgcn_permlane32_swap(x[k], x[k], false, false);
    w[k] = sw[0];
    w[4 + k] = sw[1];
  }
}

}  // namespace kvq
