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
//   2. per (group, 64-channel block): the max over the slabs' partials, the
//      scale;
//   3. per (group, slab): the codes (the keys are read a second time).
// Heads of at most kChResMaxT tokens take one launch instead: a workgroup
// per (group, 32-byte column of the rows) holds its column of every token
// in registers, so the keys are read once (channel_quantize_resident_kernel).
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

// Pass 2: scales of 64 channels of one group from the slabs' maxima.  A
// workgroup per (group, 64-channel block): lane l takes channel 64 b + l
// (each wave instruction reads 256 consecutive bytes of one slab's row of
// maxima), the 16 waves take every 16th slab with 8 slabs' loads in flight,
// and the waves' maxima meet in LDS; so a head of nslab slabs costs about
// nslab / 128 memory round trips instead of nslab / 8.
constexpr int kChScaleThreads = 1024;
constexpr int kChScaleWaves = kChScaleThreads / 64;

__global__ __launch_bounds__(kChScaleThreads) void channel_scale_kernel(
    const uint32_t* __restrict__ partials, int d, int64_t nslab, float* __restrict__ scales) {
  __shared__ uint32_t red[kChScaleWaves][64];
  const int nb = (d + 63) / 64;
  const int64_t g = blockIdx.x / nb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = (int)(blockIdx.x % nb) * 64 + lane;
  uint32_t a = 0;
  if (c < d) {
    const uint32_t* p = partials + g * nslab * d + c;
    for (int64_t s0 = w; s0 < nslab; s0 += 8 * kChScaleWaves) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t sl = s0 + (int64_t)u * kChScaleWaves;
        v[u] = sl < nslab ? p[sl * d] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) a = max(a, v[u]);
    }
  }
  red[w][lane] = a;
  __syncthreads();
  if (w == 0 && c < d) {
#pragma unroll
    for (int i = 1; i < kChScaleWaves; ++i) a = max(a, red[i][lane]);
    scales[g * d + c] = __builtin_bit_cast(float, a) / 127.0f;
  }
}

// Codes of one 16-byte chunk of a row (N channels, each with its own
// divisor sd and reciprocal rc): the quotients by reciprocal, and the
// divisions for the whole chunk where any of them could round differently
// (as the per-row quantizer: for a divisor in [2^-120, 2^120],
// |x * rcp(s) - RN32(x / s)| < 2.7e-5 since |x / s| <= 127 + 2^-16, so the
// codes agree unless x * rcp(s) lies within 2^-14 of a half-integer), or
// where a channel's reciprocal is not trusted.  The division is the
// definition, so dividing a whole chunk changes no code; one decision per
// chunk keeps the common path free of per-element branches.
template <typename T, int N = ChChunk<T>::N>
__device__ __forceinline__ typename ChChunk<T>::Codes channel_codes(const typename ChChunk<T>::V& v,
                                                                   const float (&sd)[N],
                                                                   const float (&rc)[N],
                                                                   bool untrusted) {
  float c[N];
  float dmax = 0.0f;  // largest |q - rint(q)| of the chunk (a NaN q counts as 0)
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float q = (float)v[e] * rc[e];
    c[e] = __builtin_rintf(q);
    dmax = __builtin_fmaxf(dmax, __builtin_fabsf(q - c[e]));
  }
  if (untrusted || dmax > 0.5f - 0x1p-14f) {
    // (an opaque statement keeps the divisions behind the branch)
    __asm__ volatile("");
#pragma unroll
    for (int e = 0; e < N; ++e) c[e] = __builtin_rintf((float)v[e] / sd[e]);
  }
  uint32_t w[N / 4];
#pragma unroll
  for (int h = 0; h < N / 4; ++h) {
    w[h] = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[h] |= ((uint32_t)(int)__builtin_amdgcn_fmed3f(c[4 * h + e], -128.0f, 127.0f) & 0xFFu) << (8 * e);
  }
  if constexpr (N == 4) {
    return w[0];
  } else {
    return u32x2{w[0], w[1]};
  }
}

// Divisors of N consecutive channels from their scales: a zero scale
// divides by 1; reciprocals of divisors outside [2^-120, 2^120] are not
// trusted (`untrusted` is set if any of the N is).
template <int N>
__device__ __forceinline__ void channel_divisors(const float* s, float (&sd)[N], float (&rc)[N],
                                                 bool& untrusted) {
  untrusted = false;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    sd[e] = (s[e] == 0.0f) ? 1.0f : s[e];
    rc[e] = __builtin_amdgcn_rcpf(sd[e]);
    untrusted |= !(sd[e] >= 0x1p-120f && sd[e] <= 0x1p120f);
  }
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
                    bool dv) { return channel_codes<T>(v, sd, rc, dv); };
  auto divisors = [&](int chunk, float (&sd)[N], float (&rc)[N], bool& dv) {
    channel_divisors<N>(sg + chunk * N, sd, rc, dv);
  };
  if (kChThreads % cpr == 0) {
    const int chunk = threadIdx.x % cpr;
    const int step = kChThreads / cpr;
    float sd[N], rc[N];
    bool dv;
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
      bool dv;
      divisors(chunk, sd, rc, dv);
      const typename C::V v = *reinterpret_cast<const typename C::V*>(xg + (int64_t)rr * d + chunk * N);
      *reinterpret_cast<typename C::Codes*>(cg + (int64_t)rr * d + chunk * N) = encode(v, sd, rc, dv);
    }
  }
}

// One launch for heads of at most kChResMaxT tokens.  Workgroup (g, col)
// owns 16-byte chunks 2 col and 2 col + 1 of every row of group g: lane l of
// wave w takes chunk 2 col + l / 32 of rows 256 u + 32 w + l % 32, R rows
// per lane, all in registers.  The column maxima (a 32-lane max per chunk,
// then over the 8 waves in LDS) give the scales, and the codes are encoded
// from the same registers.  Rows past the head's end re-read its last row
// (the max is unchanged) and are not stored.  When the group count is a
// multiple of 8 the workgroups of one group are placed on one XCD
// (workgroups go to XCDs round-robin), so a key line shared by several of
// them is fetched into that XCD's L2 once.
constexpr int kChResThreads = 512;
constexpr int kChResRows = kChResThreads / 2;    // rows per load step
constexpr int kChResMaxT = 16 * kChResRows;

template <typename T, int R>
__global__ __launch_bounds__(kChResThreads) void channel_quantize_resident_kernel(
    const T* __restrict__ x, int64_t groups, int64_t Ttok, int d, int8_t* __restrict__ codes,
    float* __restrict__ scales) {
  using C = ChChunk<T>;
  constexpr int N = C::N;
  __shared__ uint32_t wmax[kChResThreads / 64][2][N];
  __shared__ float wsc[2][N];
  const int nc = d / (2 * N);                      // workgroups per group
  const int64_t b = blockIdx.x;
  int64_t g;
  int col;
  if ((groups & 7) == 0) {
    const int64_t j = b >> 3;
    col = (int)(j % nc);
    g = (j / nc) * 8 + (b & 7);
  } else {
    col = (int)(b % nc);
    g = b / nc;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5;
  const int chunk = 2 * col + h;
  const int row0 = wave * 32 + (lane & 31);
  const int last = (int)Ttok - 1;
  const T* xg = x + g * Ttok * d + chunk * N;
  typename C::V v[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int r = min(u * kChResRows + row0, last);
    v[u] = *reinterpret_cast<const typename C::V*>(xg + (int64_t)r * d);
  }
  uint32_t mx[N];
#pragma unroll
  for (int e = 0; e < N; ++e) mx[e] = 0;
#pragma unroll
  for (int u = 0; u < R; ++u)
#pragma unroll
    for (int e = 0; e < N; ++e) mx[e] = max(mx[e], abs_bits((float)v[u][e]));
#pragma unroll
  for (int e = 0; e < N; ++e) mx[e] = seg_max_u32<32>(mx[e]);
  if ((lane & 31) == 0) {
#pragma unroll
    for (int e = 0; e < N; ++e) wmax[wave][h][e] = mx[e];
  }
  __syncthreads();
  if (threadIdx.x < 2 * N) {
    const int hh = threadIdx.x / N, e = threadIdx.x % N;
    uint32_t a = 0;
#pragma unroll
    for (int w = 0; w < kChResThreads / 64; ++w) a = max(a, wmax[w][hh][e]);
    const float sc = __builtin_bit_cast(float, a) / 127.0f;
    wsc[hh][e] = sc;
    scales[g * d + (2 * col + hh) * N + e] = sc;
  }
  __syncthreads();
  float sd[N], rc[N];
  bool dv;
  channel_divisors<N>(wsc[h], sd, rc, dv);
  int8_t* cg = codes + g * Ttok * d + chunk * N;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int r = u * kChResRows + row0;
    const typename C::Codes cw = channel_codes<T>(v[u], sd, rc, dv);
    if (r <= last) *reinterpret_cast<typename C::Codes*>(cg + (int64_t)r * d) = cw;
  }
}

template <typename T, int R>
static hipError_t quantize_channel_resident(const T* x, int64_t groups, int64_t Ttok, int d,
                                            int8_t* codes, float* scales, hipStream_t st) {
  const int nc = d / (2 * ChChunk<T>::N);
  // slices of whole groups, a multiple of 8 of them, so grid.x stays far
  // below 2^32 and the XCD placement holds within each slice
  const int64_t max_groups = std::max<int64_t>(8, ((int64_t(1) << 22) / nc) & ~int64_t(7));
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    hipLaunchKernelGGL((channel_quantize_resident_kernel<T, R>), dim3((unsigned)(ng * nc)),
                       dim3(kChResThreads), 0, st, x + g0 * Ttok * d, ng, Ttok, d,
                       codes + g0 * Ttok * d, scales + g0 * d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T>
static hipError_t quantize_channel_typed(const T* x, int64_t groups, int64_t Ttok, int d,
                                         int8_t* codes, float* scales, hipStream_t st) {
  static_assert(kChResThreads / 64 == 8 && kChResRows == 256, "row schedule of the resident kernel");
  if (Ttok <= kChResRows * 2)
    return quantize_channel_resident<T, 2>(x, groups, Ttok, d, codes, scales, st);
  if (Ttok <= kChResRows * 4)
    return quantize_channel_resident<T, 4>(x, groups, Ttok, d, codes, scales, st);
  if (Ttok <= kChResRows * 8)
    return quantize_channel_resident<T, 8>(x, groups, Ttok, d, codes, scales, st);
  if (Ttok <= kChResMaxT)
    return quantize_channel_resident<T, 16>(x, groups, Ttok, d, codes, scales, st);
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
      hipLaunchKernelGGL(channel_scale_kernel, dim3((unsigned)(ng * ((d + 63) / 64))),
                         dim3(kChScaleThreads), 0, st, pp, d, nslab, sp);
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
