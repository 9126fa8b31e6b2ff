// Compress-on-write for one decode step on gfx950: the newest key and value
// of every (batch, head) group are compressed and written straight into
// position `pos` of the group's compressed cache, in one launch.
//
// Keys: QJL sketch (arXiv 2406.03482, abstract): the signs of the Gaussian
// JL projection S k, packed LSB-first into 32-bit words, and the key norm.
// Values: per-row symmetric INT8 (Q-TensorFormer model card, section 6),
// encoded with the same helpers as the standalone quantizer, so the codes
// and scale are bit-identical to kvq_quantize_int8 of the same row.
//
// A workgroup takes kAppendTok groups; their keys are staged in LDS as
// binary32 and their values are quantized one row per wave in registers.
// Projections (fp16 S, d <= 128, m <= 256): each wave reads 64 rows of S with
// coalesced 1 KiB loads (4 rows per instruction, 16 lanes per row), forms
// each lane's 8 products per key and sums a row's 16 lanes with DPP; a wave
// ballot turns 64 projection signs into two sign words.  Other shapes: each
// thread owns up to four rows of S and accumulates binary32 fused
// multiply-adds in channel order.
#include "kvq_device.h"
#include "kvq_int8_device.h"
#include "kvq_launch.h"
#include "kvq_qjl_device.h"

#include <algorithm>

namespace kvq {

constexpr int kAppendTok = 2;   // 512 groups: 6.3 us against 7.7 us with 4
constexpr int kAppendThreads = 256;
constexpr int kAppendWaves = kAppendThreads / 64;
constexpr int kAppendVals = kMaxDecodeD / 64;   // value elements per lane

template <typename T>
__global__ __launch_bounds__(kAppendThreads) void cache_append_kernel(
    const T* __restrict__ k, const T* __restrict__ v, int64_t groups, int d,
    const T* __restrict__ S, int m, int64_t Tcap, int64_t pos, uint32_t* __restrict__ kbits,
    uint16_t* __restrict__ knorms, int8_t* __restrict__ vcodes, float* __restrict__ vscales) {
  __shared__ __align__(16) float ks[kAppendTok * kMaxDecodeD];   // [token][d], binary32
  const int64_t g0 = (int64_t)blockIdx.x * kAppendTok;
  const int ntok = (int)std::min<int64_t>(kAppendTok, groups - g0);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int words = m / 32;

  // fp16 S with d <= 128 and m <= 256: coalesced projection (see below); its
  // S loads are issued first so they overlap the staging of keys and values
  constexpr bool kHalf = sizeof(T) == 2;
  const bool fast = kHalf && d <= 128 && m <= kAppendThreads;
  const int c = lane & 15;
  const int r4 = lane >> 4;
  const int cc = min(c, d / 8 - 1);
  f16x8 raw[16];
  if constexpr (kHalf) {
    if (fast) {
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int row = min(64 * wave + 16 * r4 + it, m - 1);
        raw[it] = *reinterpret_cast<const f16x8*>(S + (int64_t)row * d + 8 * cc);
      }
    }
  }

  for (int i = threadIdx.x; i < ntok * d; i += kAppendThreads) ks[i] = to_f32(k[g0 * d + i]);

  // values: one row per wave
  for (int tok = wave; tok < ntok; tok += kAppendWaves) {
    const T* vr = v + (g0 + tok) * d;
    const int64_t row = (g0 + tok) * Tcap + pos;
    float x[kAppendVals];
    uint32_t amax = 0;
#pragma unroll
    for (int e = 0; e < kAppendVals; ++e) {
      const int j = lane + 64 * e;
      x[e] = j < d ? to_f32(vr[j]) : 0.0f;
      amax = max(amax, abs_bits(x[e]));
    }
    amax = seg_max_u32<64>(amax);
    const float s = row_scale(amax);
    const float sdiv = row_divisor(s);
#pragma unroll
    for (int e = 0; e < kAppendVals; ++e) {
      const int j = lane + 64 * e;
      if (j < d) vcodes[row * d + j] = (int8_t)code_of(x[e], sdiv);
    }
    if (lane == 0) vscales[row] = s;
  }
  __syncthreads();

  // key norms: one row per wave
  for (int tok = wave; tok < ntok; tok += kAppendWaves) {
    const float* kr = ks + tok * d;
    float ss = 0.0f;
    for (int j = lane; j < d; j += 64) ss = __builtin_fmaf(kr[j], kr[j], ss);
    ss = seg_sum_f32<64>(ss);
    if (lane == 0) knorms[(g0 + tok) * Tcap + pos] = f32_to_f16_bits(__builtin_sqrtf(ss));
  }

  if constexpr (kHalf) {
    if (fast) {
      // Iteration it: the wave's load read rows 64 w + 16 r4 + it (lanes of
      // segment r4, 16 bytes each); the 16 lanes of a segment sum the row's
      // products with DPP, and lane c keeps the sign of the row it == c.  A
      // ballot then yields the signs of rows 64 w .. 64 w + 63 in lane order,
      // i.e. two sign words.
      const bool live_c = 8 * c < d;
      bool sgn[kAppendTok];
#pragma unroll
      for (int u = 0; u < kAppendTok; ++u) sgn[u] = false;
#pragma unroll
      for (int u = 0; u < kAppendTok; ++u) {
        if (u >= ntok) break;
        float kv[8];
        const f32x4* p4 = reinterpret_cast<const f32x4*>(ks + u * d + 8 * cc);
        const f32x4 k0 = p4[0], k1 = p4[1];
        kv[0] = k0[0]; kv[1] = k0[1]; kv[2] = k0[2]; kv[3] = k0[3];
        kv[4] = k1[0]; kv[5] = k1[1]; kv[6] = k1[2]; kv[7] = k1[3];
#pragma unroll
        for (int it = 0; it < 16; ++it) {
          float part = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)raw[it][e], kv[e], part);
          part = seg_sum_f32<16>(live_c ? part : 0.0f);
          sgn[u] = (it == c) ? (part >= 0.0f) : sgn[u];
        }
      }
      const int row = 64 * wave + 16 * r4 + c;
      const int w0 = 2 * wave;
#pragma unroll
      for (int u = 0; u < kAppendTok; ++u) {
        if (u >= ntok) break;
        const uint64_t bal = __ballot(row < m && sgn[u]);
        uint32_t* dst = kbits + ((g0 + u) * Tcap + pos) * words;
        if (lane == 0 && w0 < words) dst[w0] = (uint32_t)bal;
        if (lane == 1 && w0 + 1 < words) dst[w0 + 1] = (uint32_t)(bal >> 32);
      }
      return;
    }
  }

  // projections: thread t owns rows t + 256 r
  float acc[kProjMaxRowsPerThread][kAppendTok];
#pragma unroll
  for (int r = 0; r < kProjMaxRowsPerThread; ++r)
#pragma unroll
    for (int u = 0; u < kAppendTok; ++u) acc[r][u] = 0.0f;
#pragma unroll
  for (int r = 0; r < kProjMaxRowsPerThread; ++r) {
    const int i = threadIdx.x + kAppendThreads * r;
    if (i < m) {
      const T* sr = S + (int64_t)i * d;
      for (int j = 0; j < d; j += 16) {
        float sv[16];
        load16_f32<T>(sr + j, sv);
#pragma unroll
        for (int u = 0; u < kAppendTok; ++u) {
          const f32x4* kv4 = reinterpret_cast<const f32x4*>(ks + u * d + j);
          float a = acc[r][u];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 kk = kv4[q4];
            a = __builtin_fmaf(sv[4 * q4 + 0], kk[0], a);
            a = __builtin_fmaf(sv[4 * q4 + 1], kk[1], a);
            a = __builtin_fmaf(sv[4 * q4 + 2], kk[2], a);
            a = __builtin_fmaf(sv[4 * q4 + 3], kk[3], a);
          }
          acc[r][u] = a;
        }
      }
    }
  }

  // sign words: a wave's 64 rows of block r are words (256 r + 64 wave) / 32 + {0, 1}
#pragma unroll
  for (int r = 0; r < kProjMaxRowsPerThread; ++r) {
    if (kAppendThreads * r >= m) break;
    const int i = threadIdx.x + kAppendThreads * r;
    const int w0 = (kAppendThreads * r + 64 * wave) / 32;
#pragma unroll
    for (int u = 0; u < kAppendTok; ++u) {
      if (u >= ntok) break;
      const uint64_t bal = __ballot(i < m && acc[r][u] >= 0.0f);
      uint32_t* dst = kbits + ((g0 + u) * Tcap + pos) * words;
      if (lane == 0 && w0 < words) dst[w0] = (uint32_t)bal;
      if (lane == 1 && w0 + 1 < words) dst[w0 + 1] = (uint32_t)(bal >> 32);
    }
  }
}

hipError_t launch_cache_append(const void* k, const void* v, int kv_f16, int64_t groups, int d,
                               const void* S, int m, int64_t T, int64_t pos, uint32_t* kbits,
                               uint16_t* knorms, int8_t* vcodes, float* vscales, hipStream_t st) {
  const int64_t max_blocks = int64_t(1) << 30;
  for (int64_t g0 = 0; g0 < groups; g0 += max_blocks * kAppendTok) {
    const int64_t ng = std::min(max_blocks * kAppendTok, groups - g0);
    const unsigned blocks = (unsigned)((ng + kAppendTok - 1) / kAppendTok);
    const int64_t off = g0 * T;                    // first cache row of the slice
    if (kv_f16)
      hipLaunchKernelGGL(cache_append_kernel<_Float16>, dim3(blocks), dim3(kAppendThreads), 0, st,
                         static_cast<const _Float16*>(k) + g0 * d,
                         static_cast<const _Float16*>(v) + g0 * d, ng, d,
                         static_cast<const _Float16*>(S), m, T, pos, kbits + off * (m / 32),
                         knorms + off, vcodes + off * d, vscales + off);
    else
      hipLaunchKernelGGL(cache_append_kernel<float>, dim3(blocks), dim3(kAppendThreads), 0, st,
                         static_cast<const float*>(k) + g0 * d,
                         static_cast<const float*>(v) + g0 * d, ng, d,
                         static_cast<const float*>(S), m, T, pos, kbits + off * (m / 32),
                         knorms + off, vcodes + off * d, vscales + off);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvq
