// Per-channel symmetric INT8 for a key cache, for gfx950.
//
// Method: the symmetric INT8 formula of the Q-TensorFormer model card
// (section 6), which the card labels channel-wise: per group g (one head)
// of keys x [T, d], the scale of channel c is max_t |x_tc| / 127 and a code
// is the nearest integer of x / scale clamped to [-128, 127].  Arithmetic as
// the per-row quantizer: s = RN32(a / 127) and x / s IEEE binary32
// divisions, rint ties to even, a zero scale gives codes 0 (divisor 1).
//
// The scale is a reduction over tokens, i.e. down the columns of row-major
// keys, so quantization takes two passes over the keys:
//   1. per (group, slab of kChSlab tokens): the slab's column max |x| (lanes
//      keep running maxima of their 16-byte chunk over the slab's rows, then
//      an LDS atomic max per channel), written as binary32 bit patterns
//      into the code buffer, which is free until pass 3 (the partials need
//      4 * ceil(T / kChSlab) <= T bytes per channel; for T <= kChSlab pass 1
//      writes the scales directly and pass 2 is skipped);
//   2. per (group, channel): the max over the slabs' partials, the scale;
//   3. per (group, slab): the codes (the keys are read a second time).
// Dequantize is a flat stream; the score folds the channel scales into the
// query (q_c s_c, one binary32 product) inside the INT8 score kernel.
#include "kvq_device.h"
#include "kvq_launch.h"

#include <algorithm>
#include <type_traits>

namespace kvq {

constexpr int kChSlab = 128;      // tokens per workgroup in passes 1 and 3 (5 % faster than 256 on a Llama-7B layer)
constexpr int kChThreads = 256;

template <typename T> struct ChChunk;
template <> struct ChChunk<float> {
  static constexpr int N = 4;
  using V = f32x4;
  using Codes = uint32_t;
};
template <> struct ChChunk<_Float16> {
  static constexpr int N = 8;
  using V = f16x8;
  using Codes = u32x2;
};

// Pass 1.  256 / cpr rows in parallel when cpr = d / N divides 256 (each
// thread owns one chunk column), else a strided walk over (row, chunk)
// pairs.  Rows past the slab's end re-read its last row (a max is
// unchanged by repeats), so the loads are unconditional.
template <typename T>
__global__ __launch_bounds__(kChThreads) void channel_absmax_kernel(
    const T* __restrict__ x, int64_t Ttok, int d, int64_t nslab, uint32_t* __restrict__ partials,
    float* __restrict__ scales) {
  using C = ChChunk<T>;
  constexpr int N = C::N;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  uint32_t* pm = reinterpret_cast<uint32_t*>(lds_raw);
  const int64_t g = blockIdx.x / nslab;
  const int64_t slab = blockIdx.x % nslab;
  const int64_t t0 = slab * kChSlab;
  const int nrows = (int)std::min<int64_t>(kChSlab, Ttok - t0);
  const int cpr = d / N;
  const T* xg = x + (g * Ttok + t0) * d;
  for (int c = threadIdx.x; c < d; c += kChThreads) pm[c] = 0;
  __syncthreads();
  if (kChThreads % cpr == 0) {
    const int chunk = threadIdx.x % cpr;
    const int step = kChThreads / cpr;
    uint32_t m[N];
#pragma unroll
    for (int e = 0; e < N; ++e) m[e] = 0;
    for (int r = threadIdx.x / cpr; r < nrows; r += 4 * step) {
      typename C::V v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = min(r + u * step, nrows - 1);
        v[u] = ld_stream(reinterpret_cast<const typename C::V*>(xg + (int64_t)rr * d + chunk * N));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < N; ++e) m[e] = max(m[e], abs_bits((float)v[u][e]));
    }
    if (threadIdx.x / cpr < nrows) {
#pragma unroll
      for (int e = 0; e < N; ++e) atomicMax(&pm[chunk * N + e], m[e]);
    }
  } else {
    for (int idx = threadIdx.x; idx < nrows * cpr; idx += kChThreads) {
      const int rr = idx / cpr, chunk = idx % cpr;
      const typename C::V v = *reinterpret_cast<const typename C::V*>(xg + (int64_t)rr * d + chunk * N);
#pragma unroll
      for (int e = 0; e < N; ++e) atomicMax(&pm[chunk * N + e], abs_bits((float)v[e]));
    }
  }
  __syncthreads();
  if (nslab == 1) {
    for (int c = threadIdx.x; c < d; c += kChThreads)
      scales[g * d + c] = __builtin_bit_cast(float, pm[c]) / 127.0f;
  } else {
    uint32_t* out = partials + (g * nslab + slab) * d;
    for (int c = threadIdx.x; c < d; c += kChThreads) out[c] = pm[c];
  }
}

// Pass 2: scale of channel c of group g from the slabs' maxima.
__global__ __launch_bounds__(kChThreads) void channel_scale_kernel(
    const uint32_t* __restrict__ partials, int64_t groups, int d, int64_t nslab,
    float* __restrict__ scales) {
  const int64_t idx = (int64_t)blockIdx.x * kChThreads + threadIdx.x;
  if (idx >= groups * d) return;
  const int64_t g = idx / d;
  const int c = (int)(idx % d);
  const uint32_t* p = partials + g * nslab * d + c;
  uint32_t a = 0;
  // 8 slabs' loads in flight at a time (past the last slab: the last one again)
  for (int64_t s0 = 0; s0 < nslab; s0 += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[std::min<int64_t>(s0 + u, nslab - 1) * d];
#pragma unroll
    for (int u = 0; u < 8; ++u) a = max(a, v[u]);
  }
  scales[idx] = __builtin_bit_cast(float, a) / 127.0f;
}

// One code for a channel's divisor: the quotient by reciprocal, divided
// only where it could round differently (as the per-row quantizer: for a
// divisor in [2^-120, 2^120], |x * rcp(s) - RN32(x / s)| < 2.7e-5 since
// |x / s| <= 127 + 2^-16, so the codes agree unless x * rcp(s) lies within
// 2^-14 of a half-integer).
__device__ __forceinline__ uint32_t channel_code(float x, float sdiv, float r, bool divide) {
  const float q = x * r;
  float c = __builtin_rintf(q);
  if (divide || __builtin_fabsf(q - c) > 0.5f - 0x1p-14f) {
    __asm__ volatile("");
    c = __builtin_rintf(x / sdiv);
  }
  return (uint32_t)(int)__builtin_amdgcn_fmed3f(c, -128.0f, 127.0f) & 0xFFu;
}

// Pass 3: codes of one slab.
template <typename T>
__global__ __launch_bounds__(kChThreads) void channel_quantize_kernel(
    const T* __restrict__ x, int64_t Ttok, int d, int64_t nslab, const float* __restrict__ scales,
    int8_t* __restrict__ codes) {
  using C = ChChunk<T>;
  constexpr int N = C::N;
  const int64_t g = blockIdx.x / nslab;
  const int64_t slab = blockIdx.x % nslab;
  const int64_t t0 = slab * kChSlab;
  const int nrows = (int)std::min<int64_t>(kChSlab, Ttok - t0);
  const int cpr = d / N;
  const T* xg = x + (g * Ttok + t0) * d;
  int8_t* cg = codes + (g * Ttok + t0) * d;
  const float* sg = scales + g * d;
  auto encode = [&](const typename C::V& v, const float (&sd)[N], const float (&rc)[N],
                    const bool (&dv)[N]) {
    typename C::Codes out;
    if constexpr (N == 4) {
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) w |= channel_code(v[e], sd[e], rc[e], dv[e]) << (8 * e);
      out = w;
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w |= channel_code((float)v[4 * h + e], sd[4 * h + e], rc[4 * h + e], dv[4 * h + e]) << (8 * e);
        out[h] = w;
      }
    }
    return out;
  };
  auto divisors = [&](int chunk, float (&sd)[N], float (&rc)[N], bool (&dv)[N]) {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const float s = sg[chunk * N + e];
      sd[e] = (s == 0.0f) ? 1.0f : s;
      rc[e] = __builtin_amdgcn_rcpf(sd[e]);
      dv[e] = !(sd[e] >= 0x1p-120f && sd[e] <= 0x1p120f);
    }
  };
  if (kChThreads % cpr == 0) {
    const int chunk = threadIdx.x % cpr;
    const int step = kChThreads / cpr;
    float sd[N], rc[N];
    bool dv[N];
    divisors(chunk, sd, rc, dv);
    for (int r = threadIdx.x / cpr; r < nrows; r += 4 * step) {
      typename C::V v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = min(r + u * step, nrows - 1);
        v[u] = ld_stream(reinterpret_cast<const typename C::V*>(xg + (int64_t)rr * d + chunk * N));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int rr = r + u * step;
        const typename C::Codes cw = encode(v[u], sd, rc, dv);
        if (rr < nrows) *reinterpret_cast<typename C::Codes*>(cg + (int64_t)rr * d + chunk * N) = cw;
      }
    }
  } else {
    for (int idx = threadIdx.x; idx < nrows * cpr; idx += kChThreads) {
      const int rr = idx / cpr, chunk = idx % cpr;
      float sd[N], rc[N];
      bool dv[N];
      divisors(chunk, sd, rc, dv);
      const typename C::V v = *reinterpret_cast<const typename C::V*>(xg + (int64_t)rr * d + chunk * N);
      *reinterpret_cast<typename C::Codes*>(cg + (int64_t)rr * d + chunk * N) = encode(v, sd, rc, dv);
    }
  }
}

template <typename T>
static hipError_t quantize_channel_typed(const T* x, int64_t groups, int64_t Ttok, int d,
                                         int8_t* codes, float* scales, hipStream_t st) {
  const int64_t nslab = (Ttok + kChSlab - 1) / kChSlab;
  const size_t lds = (size_t)d * sizeof(uint32_t);
  // launch in slices of whole groups so grid.x stays far below 2^32
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / nslab);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    const T* xp = x + g0 * Ttok * d;
    int8_t* cp = codes + g0 * Ttok * d;
    uint32_t* pp = reinterpret_cast<uint32_t*>(cp);
    float* sp = scales + g0 * d;
    hipLaunchKernelGGL((channel_absmax_kernel<T>), dim3((unsigned)(ng * nslab)), dim3(kChThreads),
                       lds, st, xp, Ttok, d, nslab, pp, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (nslab > 1) {
      const int64_t n = ng * d;
      hipLaunchKernelGGL(channel_scale_kernel, dim3((unsigned)((n + kChThreads - 1) / kChThreads)),
                         dim3(kChThreads), 0, st, pp, ng, d, nslab, sp);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((channel_quantize_kernel<T>), dim3((unsigned)(ng * nslab)), dim3(kChThreads),
                       0, st, xp, Ttok, d, nslab, sp, cp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_int8_channel(const void* x, int x_f16, int64_t groups, int64_t T, int d,
                                        int8_t* codes, float* scales, hipStream_t s) {
  if (x_f16)
    return quantize_channel_typed(static_cast<const _Float16*>(x), groups, T, d, codes, scales, s);
  return quantize_channel_typed(static_cast<const float*>(x), groups, T, d, codes, scales, s);
}

// ---------------------------------------------------------------------------
// Dequantize: flat stream of 16-byte output chunks; chunk i holds outputs
// i N .. i N + N - 1, of row i N / d and channels (i N) mod d ...
template <typename TO> struct ChOut;
template <> struct ChOut<float> {
  static constexpr int N = 4;
  using V = f32x4;
  using Codes = uint32_t;
};
template <> struct ChOut<_Float16> {
  static constexpr int N = 8;
  using V = f16x8;
  using Codes = u32x2;
};

template <typename TO>
__global__ __launch_bounds__(256) void channel_dequantize_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ scales, int64_t nchunks,
    int64_t Ttok, int d, TO* __restrict__ out) {
  using C = ChOut<TO>;
  constexpr int N = C::N;
  constexpr int U = 4;
  const int64_t base = (int64_t)blockIdx.x * (256 * U) + threadIdx.x;
  typename C::Codes cv[U];
  float sv[U][N];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = std::min<int64_t>(base + 256 * u, nchunks - 1);
    const int64_t e0 = i * N;
    const int64_t g = e0 / (Ttok * d);
    const int c0 = (int)(e0 % d);
    cv[u] = ld_stream(reinterpret_cast<const typename C::Codes*>(codes + e0));
#pragma unroll
    for (int v4 = 0; v4 < N / 4; ++v4) {
      const f32x4 sc = *reinterpret_cast<const f32x4*>(scales + g * d + c0 + 4 * v4);
      sv[u][4 * v4] = sc[0]; sv[u][4 * v4 + 1] = sc[1]; sv[u][4 * v4 + 2] = sc[2]; sv[u][4 * v4 + 3] = sc[3];
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + 256 * u;
    typename C::V o;
    if constexpr (N == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = i8_to_f32(cv[u], e) * sv[u][e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (_Float16)(i8_to_f32(cv[u][e >> 2], e & 3) * sv[u][e]);
    }
    if (i < nchunks) *reinterpret_cast<typename C::V*>(out + i * N) = o;
  }
}

hipError_t launch_dequantize_int8_channel(const int8_t* codes, const float* scales, int64_t groups,
                                          int64_t T, int d, void* out, int out_f16,
                                          hipStream_t s) {
  auto run = [&](auto* o, int N) {
    using TO = std::remove_pointer_t<decltype(o)>;
    const int64_t nchunks = groups * T * d / N;
    const int64_t blocks = (nchunks + 1023) / 1024;
    hipLaunchKernelGGL(channel_dequantize_kernel<TO>, dim3((unsigned)blocks), dim3(256), 0, s,
                       codes, scales, nchunks, T, d, o);
    return hipGetLastError();
  };
  if (out_f16) return run(static_cast<_Float16*>(out), 8);
  return run(static_cast<float*>(out), 4);
}

}  // namespace kvq
