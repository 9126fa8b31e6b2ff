// Asymmetric group-wise INT4 quantize / dequantize for gfx950.
//
// Method: the asymmetric group-wise INT4 formula of the Q-TensorFormer model
// card (section 6, "Adaptive KV Cache Quantization & Attention-Sink
// Eviction"): over a group of values the step is (max - min) / 15 and the
// offset is the minimum; a code is the nearest integer of (x - offset) /
// step clamped to [0, 15]; the reconstruction is code * step + offset.
//
// Arithmetic (bit-exact): s = RN32(RN32(max - min) / 15), z = min,
// code = med3(rint(RN32(RN32(x - z) / s)), 0, 15) with IEEE binary32
// subtraction and division (no fast-math, subnormals kept, rint = ties to
// even); x_hat = RN32(RN32(code * s) + z), never contracted to an fma.  A
// group whose step is +0 gets all-zero codes (divisor 1: every x - z of such
// a group is below 15 * 2^-150, so its rint is 0).  The quantizer of
// power-of-two groups multiplies by a reciprocal instead of dividing and
// divides only where that could change a code (encode4_rcp below).
//
// Layout: groups are g consecutive values of a row and rows are contiguous,
// so the whole tensor is a flat sequence of rows * d / g groups; codes are
// two per byte (even element in the low nibble), steps and offsets one
// binary32 each per group in group order.
//
// Memory: both kernels are HBM streams.  Lanes load 16 contiguous bytes each
// so every load instruction of a wave reads 1 KiB; group min/max are reduced
// across the lanes of a group with DPP/swizzle moves, never through LDS.
#include "kvq_device.h"
#include "kvq_int4_device.h"
#include "kvq_launch.h"

#include <algorithm>

namespace kvq {

template <typename T> struct In4;
template <> struct In4<float> {
  static constexpr int N = 4;      // elements per 16-byte chunk
  using V = f32x4;
  using Codes = uint16_t;          // 4 nibbles
};
template <> struct In4<_Float16> {
  static constexpr int N = 8;
  using V = f16x8;
  using Codes = uint32_t;          // 8 nibbles
};

template <typename T>
__device__ __forceinline__ typename In4<T>::Codes encode4(const typename In4<T>::V& v, float z,
                                                          float sdiv) {
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < In4<T>::N; ++e) w |= nibble_of((float)v[e], z, sdiv) << (4 * e);
  return (typename In4<T>::Codes)w;
}

// Same codes as encode4 with one multiply per value instead of a division
// (codes_rcp).
template <typename T>
__device__ __forceinline__ typename In4<T>::Codes encode4_rcp(const typename In4<T>::V& v, float z,
                                                              float sdiv, float r, bool divide) {
  constexpr int N = In4<T>::N;
  float x[N], c[N];
#pragma unroll
  for (int e = 0; e < N; ++e) x[e] = (float)v[e];
  codes_rcp<N>(x, z, sdiv, r, divide, c);
  return (typename In4<T>::Codes)pack_nibbles<N>(c);
}

template <typename T>
__device__ __forceinline__ void chunk_minmax(const typename In4<T>::V& v, float& mn, float& mx) {
#pragma unroll
  for (int e = 0; e < In4<T>::N; ++e) {
    mn = __builtin_fminf(mn, (float)v[e]);
    mx = __builtin_fmaxf(mx, (float)v[e]);
  }
}

// ---------------------------------------------------------------------------
// Quantize, power-of-two groups: LPG lanes per group, CPL chunks per lane and
// group (g == LPG * CPL * N), UNROLL group passes per wave in flight.  Loads
// are unconditional (groups past the end re-read the last group; nothing of
// theirs is stored).
template <typename T, int LPG, int CPL, int UNROLL>
__global__ __launch_bounds__(256) void quantize_int4_kernel(const T* __restrict__ x,
                                                            int64_t ngroups,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ steps,
                                                            float* __restrict__ offsets) {
  using C = In4<T>;
  constexpr int N = C::N;
  constexpr int G = LPG * CPL * N;
  constexpr int GPP = kWave / LPG;  // groups per wave pass
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPG;
  const int gg = lane / LPG;
  const int64_t grp0 = ((int64_t)blockIdx.x * 4 + wave) * (GPP * UNROLL) + gg;

  typename C::V v[UNROLL][CPL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t grp = std::min<int64_t>(grp0 + u * GPP, ngroups - 1);
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      v[u][j] = ld_stream(reinterpret_cast<const typename C::V*>(x + grp * G + (int64_t)(sub + LPG * j) * N));
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t grp = grp0 + u * GPP;
    float mn = (float)v[u][0][0], mx = mn;
#pragma unroll
    for (int j = 0; j < CPL; ++j) chunk_minmax<T>(v[u][j], mn, mx);
    mn = seg_min_f32<LPG>(mn);
    mx = seg_max_f32<LPG>(mx);
    const float s = group_step(mn, mx);
    const float sdiv = step_divisor(s);
    const float r = __builtin_amdgcn_rcpf(sdiv);
    const bool divide = !rcp_ok(sdiv);
    if (grp < ngroups) {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        *reinterpret_cast<typename C::Codes*>(codes + grp * (G / 2) + (int64_t)(sub + LPG * j) * (N / 2)) =
            encode4_rcp<T>(v[u][j], mn, sdiv, r, divide);
      if (sub == 0) {
        steps[grp] = s;
        offsets[grp] = mn;
      }
    }
  }
}

// Quantize, any g % 16 == 0: one group per wave, a min/max pass and a code
// pass (the second reads the group again, from cache).
template <typename T>
__global__ __launch_bounds__(256) void quantize_int4_generic_kernel(const T* __restrict__ x,
                                                                    int64_t ngroups, int g,
                                                                    uint8_t* __restrict__ codes,
                                                                    float* __restrict__ steps,
                                                                    float* __restrict__ offsets) {
  using C = In4<T>;
  constexpr int N = C::N;
  const int lane = threadIdx.x & 63;
  const int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (grp >= ngroups) return;  // uniform per wave
  const int cpg = g / N;
  const T* xg = x + grp * g;
  float mn = (float)xg[0], mx = mn;
  for (int c = lane; c < cpg; c += kWave)
    chunk_minmax<T>(*reinterpret_cast<const typename C::V*>(xg + (int64_t)c * N), mn, mx);
  mn = seg_min_f32<64>(mn);
  mx = seg_max_f32<64>(mx);
  const float s = group_step(mn, mx);
  const float sdiv = step_divisor(s);
  for (int c = lane; c < cpg; c += kWave)
    *reinterpret_cast<typename C::Codes*>(codes + grp * (g / 2) + (int64_t)c * (N / 2)) =
        encode4<T>(*reinterpret_cast<const typename C::V*>(xg + (int64_t)c * N), mn, sdiv);
  if (lane == 0) {
    steps[grp] = s;
    offsets[grp] = mn;
  }
}

template <typename T>
// ngroups: groups of this launch; total: groups of the whole call (it picks
// the passes per wave; calls are launched in slices of kGroupsPerLaunch)
static hipError_t quantize_int4_dispatch(const T* x, int64_t ngroups, int64_t total, int g,
                                         uint8_t* codes, float* steps, float* offsets,
                                         hipStream_t st) {
  constexpr int N = In4<T>::N;
  const int cpg = g / N;
  auto lanes = [&](auto kernel, int lpg, int unroll) {
    const int64_t per_block = 4LL * (kWave / lpg) * unroll;
    const int64_t blocks = (ngroups + per_block - 1) / per_block;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, ngroups, codes, steps,
                       offsets);
    return hipGetLastError();
  };
  const int64_t elems = total * g;
  const bool few_passes = sizeof(T) == 2 ? elems <= (int64_t(1) << 27) : elems > (int64_t(1) << 28);
  if ((cpg & (cpg - 1)) == 0) {
    switch (cpg) {
      case 2: return lanes(quantize_int4_kernel<T, 2, 1, 8>, 2, 8);
      // Groups of 4, 8 or 16 chunks: two group passes per wave for fp16 calls
      // of up to 2^27 elements and fp32 calls of more than 2^28, else eight
      // (measured: fp16 g = 32 / 128 on a Llama-7B layer, 2^25 elements, 6-7 %
      // faster with two, at 2^30 2-3 % slower; fp32 g = 32 / 64 at 2^30 7-9 %
      // faster with two, g = 32 at 2^28 3 % slower)
      case 4:
        return few_passes ? lanes(quantize_int4_kernel<T, 4, 1, 2>, 4, 2)
                          : lanes(quantize_int4_kernel<T, 4, 1, 8>, 4, 8);
      case 8:
        return few_passes ? lanes(quantize_int4_kernel<T, 8, 1, 2>, 8, 2)
                          : lanes(quantize_int4_kernel<T, 8, 1, 8>, 8, 8);
      case 16:
        return few_passes ? lanes(quantize_int4_kernel<T, 16, 1, 2>, 16, 2)
                          : lanes(quantize_int4_kernel<T, 16, 1, 8>, 16, 8);
      case 32: return lanes(quantize_int4_kernel<T, 16, 2, 4>, 16, 4);
      case 64: return lanes(quantize_int4_kernel<T, 64, 1, 4>, 64, 4);
      case 128: return lanes(quantize_int4_kernel<T, 64, 2, 4>, 64, 4);
      case 256: return lanes(quantize_int4_kernel<T, 64, 4, 2>, 64, 2);
      default: break;
    }
  }
  const int64_t blocks = (ngroups + 3) / 4;
  hipLaunchKernelGGL(quantize_int4_generic_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st, x,
                     ngroups, g, codes, steps, offsets);
  return hipGetLastError();
}

// Groups per launch: keeps every grid far below 2^32 threads.
constexpr int64_t kGroupsPerLaunch = int64_t(1) << 24;

template <typename T>
static hipError_t quantize_int4_sliced(const T* x, int64_t ngroups, int g, uint8_t* codes,
                                       float* steps, float* offsets, hipStream_t s) {
  for (int64_t g0 = 0; g0 < ngroups; g0 += kGroupsPerLaunch) {
    const int64_t n = std::min(kGroupsPerLaunch, ngroups - g0);
    hipError_t e = quantize_int4_dispatch(x + g0 * g, n, ngroups, g, codes + g0 * (g / 2),
                                          steps + g0, offsets + g0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_int4(const void* x, int x_f16, int64_t rows, int d, int g,
                                uint8_t* codes, float* steps, float* offsets, hipStream_t s) {
  const int64_t ngroups = rows * (d / g);
  if (x_f16)
    return quantize_int4_sliced(static_cast<const _Float16*>(x), ngroups, g, codes, steps, offsets, s);
  return quantize_int4_sliced(static_cast<const float*>(x), ngroups, g, codes, steps, offsets, s);
}

// ---------------------------------------------------------------------------
// Dequantize: a flat stream of 16-byte output chunks; chunk i holds outputs
// i * N .. i * N + N - 1 of group i * N / g.  UNROLL chunks per thread,
// consecutive threads on consecutive chunks.
template <typename TO> struct Out4;
template <> struct Out4<float> {
  static constexpr int N = 4;
  using V = f32x4;
  using Codes = uint16_t;
};
template <> struct Out4<_Float16> {
  static constexpr int N = 8;
  using V = f16x8;
  using Codes = uint32_t;
};

template <typename TO>
__device__ __forceinline__ typename Out4<TO>::V decode4(uint32_t w, float s, float z) {
  typename Out4<TO>::V out;
#pragma unroll
  for (int e = 0; e < Out4<TO>::N; ++e) out[e] = (TO)recon4((float)((w >> (4 * e)) & 0xFu), s, z);
  return out;
}

template <typename TO, int UNROLL, bool POW2>
__global__ __launch_bounds__(256) void dequantize_int4_kernel(const uint8_t* __restrict__ codes,
                                                              const float* __restrict__ steps,
                                                              const float* __restrict__ offsets,
                                                              int64_t nchunks, int cpg_shift,
                                                              int cpg, TO* __restrict__ out) {
  using C = Out4<TO>;
  constexpr int N = C::N;
  const int64_t base = (int64_t)blockIdx.x * (256 * UNROLL) + threadIdx.x;
  uint32_t cw[UNROLL];
  float sv[UNROLL], zv[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t i = std::min<int64_t>(base + 256 * u, nchunks - 1);
    const int64_t grp = POW2 ? (i >> cpg_shift) : (i / cpg);
    cw[u] = ld_stream(reinterpret_cast<const typename C::Codes*>(codes + i * (N / 2)));
    sv[u] = steps[grp];
    zv[u] = offsets[grp];
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t i = base + 256 * u;
    if (i < nchunks) *reinterpret_cast<typename C::V*>(out + i * N) = decode4<TO>(cw[u], sv[u], zv[u]);
  }
}

template <typename TO>
static hipError_t dequantize_int4_dispatch(const uint8_t* codes, const float* steps,
                                           const float* offsets, int64_t ngroups, int g, TO* out,
                                           hipStream_t st) {
  constexpr int N = Out4<TO>::N;
  // two output chunks per thread: against four, 2-5 % faster with fp16
  // output, the same with fp32 output
  constexpr int UNROLL = 2;
  const int cpg = g / N;
  const int64_t nchunks = ngroups * cpg;
  const int64_t blocks = (nchunks + 256 * UNROLL - 1) / (256 * UNROLL);
  if ((cpg & (cpg - 1)) == 0) {
    const int shift = __builtin_ctz((unsigned)cpg);
    hipLaunchKernelGGL((dequantize_int4_kernel<TO, UNROLL, true>), dim3((unsigned)blocks),
                       dim3(256), 0, st, codes, steps, offsets, nchunks, shift, cpg, out);
  } else {
    hipLaunchKernelGGL((dequantize_int4_kernel<TO, UNROLL, false>), dim3((unsigned)blocks),
                       dim3(256), 0, st, codes, steps, offsets, nchunks, 0, cpg, out);
  }
  return hipGetLastError();
}

template <typename TO>
static hipError_t dequantize_int4_sliced(const uint8_t* codes, const float* steps,
                                         const float* offsets, int64_t ngroups, int g, TO* out,
                                         hipStream_t s) {
  for (int64_t g0 = 0; g0 < ngroups; g0 += kGroupsPerLaunch) {
    const int64_t n = std::min(kGroupsPerLaunch, ngroups - g0);
    hipError_t e = dequantize_int4_dispatch(codes + g0 * (g / 2), steps + g0, offsets + g0, n, g,
                                            out + g0 * g, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_dequantize_int4(const uint8_t* codes, const float* steps, const float* offsets,
                                  int64_t rows, int d, int g, void* out, int out_f16,
                                  hipStream_t s) {
  const int64_t ngroups = rows * (d / g);
  if (out_f16)
    return dequantize_int4_sliced(codes, steps, offsets, ngroups, g, static_cast<_Float16*>(out), s);
  return dequantize_int4_sliced(codes, steps, offsets, ngroups, g, static_cast<float*>(out), s);
}

}  // namespace kvq
