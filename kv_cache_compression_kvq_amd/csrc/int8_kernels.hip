// Per-row symmetric INT8 quantize / dequantize / scale-folded score for gfx950.
//
// Method: the symmetric INT8 formula of the Q-TensorFormer model card
// (section 6, "Adaptive KV Cache Quantization & Attention-Sink Eviction"):
// the row scale is max|x| / 127, a code is the nearest integer of x / scale
// clamped to [-128, 127], the reconstruction is code * scale; applied per
// token as in the INT8 KV-cache paper (arXiv 2601.04719, Abstract).
//
// Arithmetic: s = a / 127 and t = x / s are IEEE binary32 divisions (the
// compiler's correctly rounded sequence; no fast-math, denormals kept);
// rint rounds half to even; the clamp is a med3.  The quantizers multiply by
// a reciprocal and divide only where the quotient's rounding could change a
// code (encode_chunk below): the codes are those of the division.
//
// Memory: all three kernels are HBM streams.  Lanes are mapped so that each
// load instruction of a wave reads 1 KiB of contiguous memory (16 B per
// lane); rows are reduced across lanes with DPP/swizzle, never through LDS,
// except for rows longer than one wave can hold (one row per workgroup).
#include "kvq_device.h"
#include "kvq_int8_device.h"
#include "kvq_launch.h"

#include <algorithm>

namespace kvq {

template <typename T> struct Chunk;
template <> struct Chunk<float> {
  static constexpr int N = 4;          // elements per 16-byte chunk
  using V = f32x4;
  using Codes = uint32_t;              // 4 codes
};
template <> struct Chunk<_Float16> {
  static constexpr int N = 8;
  using V = f16x8;
  using Codes = u32x2;                 // 8 codes
};

// Codes of one chunk: rint(RN32(x / s)) clamped to [-128, 127].  For s in
// [2^-120, 2^120], q = RN32(x * rcp(s)) (v_rcp_f32: within 1 ulp) differs
// from RN32(x / s) by at most 127 * (2^-23 + 2^-24) + 2^-18 < 2.7e-5
// (|x / s| <= 127 + 2^-16), so both round to the same integer unless q lies
// within 2^-14 of a half-integer; lanes with such a q, or rows whose scale
// is outside the range, divide.
template <typename T>
__device__ __forceinline__ typename Chunk<T>::Codes encode_chunk(const typename Chunk<T>::V& v,
                                                                 float sdiv) {
  constexpr int N = Chunk<T>::N;
  const float r = __builtin_amdgcn_rcpf(sdiv);
  bool near = !(sdiv >= 0x1p-120f && sdiv <= 0x1p120f);
  float c[N];
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const float q = (float)v[e] * r;
    c[e] = __builtin_rintf(q);
    near |= __builtin_fabsf(q - c[e]) > 0.5f - 0x1p-14f;
  }
  if (near) {
    // (an opaque statement keeps the divisions behind the branch)
    __asm__ volatile("");
#pragma unroll
    for (int e = 0; e < N; ++e) c[e] = __builtin_rintf((float)v[e] / sdiv);
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

template <typename T>
__device__ __forceinline__ uint32_t chunk_absmax(const typename Chunk<T>::V& v) {
  uint32_t m = 0;
#pragma unroll
  for (int e = 0; e < Chunk<T>::N; ++e) m = max(m, abs_bits((float)v[e]));
  return m;
}

// ---------------------------------------------------------------------------
// Quantize, rows shorter than a wave: LPR lanes per row, CPL 16-byte chunks
// per lane and row, UNROLL independent row passes per wave for memory-level
// parallelism.  d == LPR * CPL * N.
template <typename T, int LPR, int CPL, int UNROLL>
__global__ __launch_bounds__(256) void quantize_lanes_kernel(const T* __restrict__ x, int64_t rows,
                                                             int8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
  using C = Chunk<T>;
  constexpr int N = C::N;
  constexpr int CPR = LPR * CPL;
  constexpr int D = CPR * N;
  constexpr int RPP = kWave / LPR;  // rows per pass
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int rr = lane / LPR;
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * (RPP * UNROLL);

  typename C::V v[UNROLL][CPL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t row = row0 + u * RPP + rr;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      if (row < rows)
        v[u][j] = ld_stream(reinterpret_cast<const typename C::V*>(x + row * D + (int64_t)(sub + LPR * j) * N));
      else
        v[u][j] = typename C::V{};
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t row = row0 + u * RPP + rr;
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) m = max(m, chunk_absmax<T>(v[u][j]));
    m = seg_max_u32<LPR>(m);
    const float s = row_scale(m);
    const float sdiv = row_divisor(s);
    if (row < rows) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        *reinterpret_cast<typename C::Codes*>(codes + row * D + (int64_t)(sub + LPR * j) * N) =
            encode_chunk<T>(v[u][j], sdiv);
      }
      if (sub == 0) scales[row] = s;
    }
  }
}

// Quantize, one row per 256-thread workgroup held in registers:
// d == 256 * CPL * N.
template <typename T, int CPL>
__global__ __launch_bounds__(256) void quantize_block_kernel(const T* __restrict__ x, int64_t rows,
                                                             int8_t* __restrict__ codes,
                                                             float* __restrict__ scales) {
  using C = Chunk<T>;
  constexpr int N = C::N;
  constexpr int D = 256 * CPL * N;
  __shared__ uint32_t wave_max[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const T* xr = x + row * D;
  typename C::V v[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    v[j] = ld_stream(reinterpret_cast<const typename C::V*>(xr + (int64_t)(tid + 256 * j) * N));
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) m = max(m, chunk_absmax<T>(v[j]));
  m = seg_max_u32<64>(m);
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  m = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
  const float s = row_scale(m);
  const float sdiv = row_divisor(s);
#pragma unroll
  for (int j = 0; j < CPL; ++j)
    *reinterpret_cast<typename C::Codes*>(codes + row * D + (int64_t)(tid + 256 * j) * N) =
        encode_chunk<T>(v[j], sdiv);
  if (tid == 0) scales[row] = s;
}

// Quantize, any d % 16 == 0: one row per wave, a max pass and a code pass.
template <typename T>
__global__ __launch_bounds__(256) void quantize_generic_kernel(const T* __restrict__ x, int64_t rows,
                                                               int d, int8_t* __restrict__ codes,
                                                               float* __restrict__ scales) {
  using C = Chunk<T>;
  constexpr int N = C::N;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wave
  const int cpr = d / N;
  const T* xr = x + row * d;
  uint32_t m = 0;
  for (int c = lane; c < cpr; c += kWave)
    m = max(m, chunk_absmax<T>(*reinterpret_cast<const typename C::V*>(xr + (int64_t)c * N)));
  m = seg_max_u32<64>(m);
  const float s = row_scale(m);
  const float sdiv = row_divisor(s);
  for (int c = lane; c < cpr; c += kWave)
    *reinterpret_cast<typename C::Codes*>(codes + row * d + (int64_t)c * N) =
        encode_chunk<T>(*reinterpret_cast<const typename C::V*>(xr + (int64_t)c * N), sdiv);
  if (lane == 0) scales[row] = s;
}

template <typename T>
static hipError_t quantize_dispatch(const T* x, int64_t rows, int d, int8_t* codes, float* scales,
                                    hipStream_t st) {
  constexpr int N = Chunk<T>::N;
  const int cpr = d / N;
  const bool pow2 = (cpr & (cpr - 1)) == 0;
  auto lanes = [&](auto kernel, int lpr, int unroll) {
    const int64_t rows_per_block = 4LL * (kWave / lpr) * unroll;
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, rows, codes, scales);
    return hipGetLastError();
  };
  auto block = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)rows), dim3(256), 0, st, x, rows, codes, scales);
    return hipGetLastError();
  };
  if (pow2) {
    switch (cpr) {
      case 1: return lanes(quantize_lanes_kernel<T, 1, 1, 8>, 1, 8);
      case 2: return lanes(quantize_lanes_kernel<T, 2, 1, 8>, 2, 8);
      case 4: return lanes(quantize_lanes_kernel<T, 4, 1, 8>, 4, 8);
      case 8: return lanes(quantize_lanes_kernel<T, 8, 1, 8>, 8, 8);
      // fp16 rows of 128: two row passes per wave (more, smaller workgroups)
      // measured 13 % faster at 2^18 rows and 6 % at 2^23 than eight
      case 16:
        return sizeof(T) == 2 ? lanes(quantize_lanes_kernel<T, 16, 1, 2>, 16, 2)
                              : lanes(quantize_lanes_kernel<T, 16, 1, 8>, 16, 8);
      case 32: return lanes(quantize_lanes_kernel<T, 32, 1, 16>, 32, 16);
      case 64: return lanes(quantize_lanes_kernel<T, 64, 1, 4>, 64, 4);
      case 128: return lanes(quantize_lanes_kernel<T, 64, 2, 4>, 64, 4);
      // one row pass per wave: 4 % faster than four for fp32 d = 1024 at 2^28 and 2^30
      case 256: return lanes(quantize_lanes_kernel<T, 64, 4, 1>, 64, 1);
      case 512: return lanes(quantize_lanes_kernel<T, 64, 8, 1>, 64, 1);
      case 1024: return block(quantize_block_kernel<T, 4>);
      case 2048: return block(quantize_block_kernel<T, 8>);
      case 4096: return block(quantize_block_kernel<T, 16>);
      default: break;
    }
  }
  const int64_t blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(quantize_generic_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, st, x, rows,
                     d, codes, scales);
  return hipGetLastError();
}

// Rows per launch: keeps every grid far below 2^32 threads.
constexpr int64_t kRowsPerLaunch = int64_t(1) << 22;

template <typename T>
static hipError_t quantize_sliced(const T* x, int64_t rows, int d, int8_t* codes, float* scales,
                                  hipStream_t s) {
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = std::min(kRowsPerLaunch, rows - r0);
    hipError_t e = quantize_dispatch(x + r0 * d, nr, d, codes + r0 * d, scales + r0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_int8(const void* x, int x_f16, int64_t rows, int d, int8_t* codes,
                                float* scales, hipStream_t s) {
  if (x_f16) return quantize_sliced(static_cast<const _Float16*>(x), rows, d, codes, scales, s);
  return quantize_sliced(static_cast<const float*>(x), rows, d, codes, scales, s);
}

// ---------------------------------------------------------------------------
// Dequantize: a flat stream of 16-byte output chunks; chunk i of the output
// belongs to row i / (d / N).  UNROLL chunks per thread, consecutive threads
// on consecutive chunks.
template <typename TO> struct OutChunk;
template <> struct OutChunk<float> {
  static constexpr int N = 4;
  using V = f32x4;
  using Codes = uint32_t;
};
template <> struct OutChunk<_Float16> {
  static constexpr int N = 8;
  using V = f16x8;
  using Codes = u32x2;
};

template <typename TO>
__device__ __forceinline__ typename OutChunk<TO>::V decode_chunk(typename OutChunk<TO>::Codes c,
                                                                 float s) {
  typename OutChunk<TO>::V out;
  if constexpr (OutChunk<TO>::N == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = i8_to_f32(c, e) * s;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (_Float16)(i8_to_f32(c[e >> 2], e & 3) * s);
  }
  return out;
}

template <typename TO, int UNROLL, bool POW2>
__global__ __launch_bounds__(256) void dequantize_flat_kernel(const int8_t* __restrict__ codes,
                                                              const float* __restrict__ scales,
                                                              int64_t nchunks, int cpr_shift, int cpr,
                                                              TO* __restrict__ out) {
  using C = OutChunk<TO>;
  constexpr int N = C::N;
  const int64_t base = (int64_t)blockIdx.x * (256 * UNROLL) + threadIdx.x;
  typename C::Codes cv[UNROLL];
  float sv[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t i = base + 256 * u;
    if (i < nchunks) {
      const int64_t row = POW2 ? (i >> cpr_shift) : (i / cpr);
      cv[u] = ld_stream(reinterpret_cast<const typename C::Codes*>(codes + i * N));
      sv[u] = scales[row];
    } else {
      cv[u] = typename C::Codes{};
      sv[u] = 0.0f;
    }
  }
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const int64_t i = base + 256 * u;
    if (i < nchunks) *reinterpret_cast<typename C::V*>(out + i * N) = decode_chunk<TO>(cv[u], sv[u]);
  }
}

template <typename TO>
static hipError_t dequantize_dispatch(const int8_t* codes, const float* scales, int64_t rows, int d,
                                      TO* out, hipStream_t st) {
  constexpr int N = OutChunk<TO>::N;
  // two output chunks per thread: against four, 6-9 % faster with fp32
  // output at 2^28 / 2^30 elements and 5-9 % with fp16 output
  constexpr int UNROLL = 2;
  const int cpr = d / N;
  const int64_t nchunks = rows * cpr;
  const int64_t blocks = (nchunks + 256 * UNROLL - 1) / (256 * UNROLL);
  if ((cpr & (cpr - 1)) == 0) {
    const int shift = __builtin_ctz((unsigned)cpr);
    hipLaunchKernelGGL((dequantize_flat_kernel<TO, UNROLL, true>), dim3((unsigned)blocks), dim3(256),
                       0, st, codes, scales, nchunks, shift, cpr, out);
  } else {
    hipLaunchKernelGGL((dequantize_flat_kernel<TO, UNROLL, false>), dim3((unsigned)blocks),
                       dim3(256), 0, st, codes, scales, nchunks, 0, cpr, out);
  }
  return hipGetLastError();
}

template <typename TO>
static hipError_t dequantize_sliced(const int8_t* codes, const float* scales, int64_t rows, int d,
                                    TO* out, hipStream_t s) {
  for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
    const int64_t nr = std::min(kRowsPerLaunch, rows - r0);
    hipError_t e = dequantize_dispatch(codes + r0 * d, scales + r0, nr, d, out + r0 * d, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_dequantize_int8(const int8_t* codes, const float* scales, int64_t rows, int d,
                                  void* out, int out_f16, hipStream_t s) {
  if (out_f16)
    return dequantize_sliced(codes, scales, rows, d, static_cast<_Float16*>(out), s);
  return dequantize_sliced(codes, scales, rows, d, static_cast<float*>(out), s);
}

// ---------------------------------------------------------------------------
// Scale-folded INT8 score: 8 lanes per token, 16 codes (one 16-byte chunk)
// per lane and step; a wave covers 8 tokens per pass and UNROLL passes.  The
// block's query rows sit in LDS as binary32; queries are processed NQC at a
// time so every code chunk is converted once per NQC queries.
constexpr int kScoreLpt = 8;
constexpr int kScoreUnroll = 4;
constexpr int kScoreNqc = 4;
constexpr int kScoreTokensPerBlock = 4 * 8 * kScoreUnroll;  // 128
constexpr int kScoreLdsFloats = 8192;                       // 32 KiB of queries per pass

// Query values c*16 .. c*16+15 of query row jj, as binary32.
template <typename TQ, bool QLDS>
__device__ __forceinline__ void query_chunk(const float* qs, const TQ* qg, int d, int jj, int c,
                                            float out[16]) {
  if constexpr (QLDS) {
    const f32x4* qv = reinterpret_cast<const f32x4*>(qs + jj * d + c * 16);
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const f32x4 v = qv[e4];
      out[4 * e4 + 0] = v[0]; out[4 * e4 + 1] = v[1]; out[4 * e4 + 2] = v[2]; out[4 * e4 + 3] = v[3];
    }
  } else {
    const TQ* p = qg + (int64_t)jj * d + c * 16;
#pragma unroll
    for (int e = 0; e < 16; ++e) out[e] = to_f32(p[e]);
  }
}

// CH: per-channel scales (scales [groups, d]): the query staged in LDS is
// q_c * s_c (one binary32 product) and the token factor is 1.
template <typename TQ, bool QLDS, bool CH = false>
__global__ __launch_bounds__(256) void scores_int8_kernel(const TQ* __restrict__ q, int nq,
                                                          const int8_t* __restrict__ codes,
                                                          const float* __restrict__ scales,
                                                          int64_t T, int d, int64_t tiles,
                                                          float* __restrict__ scores) {
  __shared__ float qs[QLDS ? kScoreLdsFloats : 1];
  const int64_t g = blockIdx.x / tiles;
  const int64_t tile = blockIdx.x % tiles;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane % kScoreLpt;
  const int slot = lane / kScoreLpt;
  const int cpr = d / 16;
  const int64_t t0 = tile * kScoreTokensPerBlock + wave * (8 * kScoreUnroll);
  const int8_t* cg = codes + g * T * d;
  const int nq_pass = QLDS ? min(kScoreNqc, kScoreLdsFloats / d) : kScoreNqc;

  // Every load is unconditional (tokens past T re-read token T - 1, chunks
  // past the row re-read its last chunk; neither is used): loads under a
  // branch make the compiler wait for each one.  The scales and the first
  // chunk of codes are requested before the query is staged.
  int64_t tc[kScoreUnroll];
  float st[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u) {
    tc[u] = std::min<int64_t>(t0 + u * 8 + slot, T - 1);
    if constexpr (CH)
      st[u] = 1.0f;
    else
      st[u] = scales[g * T + tc[u]];
  }
  const int c_first = min(sub, cpr - 1);
  u32x4 w_first[kScoreUnroll];
#pragma unroll
  for (int u = 0; u < kScoreUnroll; ++u)
    w_first[u] = ld_stream(reinterpret_cast<const u32x4*>(cg + tc[u] * d + (int64_t)c_first * 16));

  for (int j0 = 0; j0 < nq; j0 += nq_pass) {
    const int nqc = min(nq_pass, nq - j0);
    const TQ* qg = q + ((int64_t)g * nq + j0) * d;
    if constexpr (QLDS) {
      __syncthreads();
      if constexpr (CH) {
        for (int i = threadIdx.x; i < nqc * d; i += 256) qs[i] = to_f32(qg[i]) * scales[g * d + i % d];
      } else {
        for (int i = threadIdx.x; i < nqc * d; i += 256) qs[i] = to_f32(qg[i]);
      }
      __syncthreads();
    }
    float acc[kScoreUnroll][kScoreNqc];
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u)
#pragma unroll
      for (int jj = 0; jj < kScoreNqc; ++jj) acc[u][jj] = 0.0f;

    for (int c = sub; c < cpr; c += kScoreLpt) {
      u32x4 w[kScoreUnroll];
#pragma unroll
      for (int u = 0; u < kScoreUnroll; ++u)
        w[u] = (j0 == 0 && c == sub)
                   ? w_first[u]
                   : ld_stream(reinterpret_cast<const u32x4*>(cg + tc[u] * d + (int64_t)c * 16));
#pragma unroll
      for (int jj = 0; jj < kScoreNqc; ++jj) {
        if (jj < nqc) {
          float qv[16];
          query_chunk<TQ, QLDS>(qs, qg, d, jj, c, qv);
#pragma unroll
          for (int u = 0; u < kScoreUnroll; ++u) {
            float a = acc[u][jj];
#pragma unroll
            for (int e = 0; e < 16; ++e) a = __builtin_fmaf(qv[e], i8_to_f32(w[u][e >> 2], e & 3), a);
            acc[u][jj] = a;
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int64_t t = t0 + u * 8 + slot;
#pragma unroll
      for (int jj = 0; jj < kScoreNqc; ++jj) {
        const float tot = seg_sum_f32<kScoreLpt>(acc[u][jj]);
        if (jj < nqc && sub == 0 && t < T) scores[((int64_t)g * nq + j0 + jj) * T + t] = tot * st[u];
      }
    }
  }
}

// Scale-folded INT8 score, d = 128, up to 4 queries per group: 8 lanes per
// token (lane `sub` owns channels 16 sub .. 16 sub + 15, its query values in
// registers), 8 tokens per wave pass, kS128U passes in flight and the next
// iteration's codes and scales requested before the current one is scored.
// Each block covers ITERS * 128 tokens of one group.  Same arithmetic as
// scores_int8_kernel (per-lane fused multiply-adds in channel order, an
// 8-lane DPP sum, then the token scale), so the same scores bit for bit.
constexpr int kS128U = 4;
constexpr int kS128Step = 4 * 8 * kS128U;                 // tokens per block iteration

template <typename TQ, int NQ, bool CH, int ITERS>
__global__ __launch_bounds__(256) void scores_int8_d128_kernel(const TQ* __restrict__ q,
                                                               const int8_t* __restrict__ codes,
                                                               const float* __restrict__ scales,
                                                               int64_t T, int64_t tiles,
                                                               float* __restrict__ scores) {
  constexpr int D = 128;
  __shared__ __align__(16) float qs[NQ * D];
  const int64_t g = blockIdx.x / tiles;
  const int64_t tile = blockIdx.x % tiles;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & 7;
  const int slot = lane >> 3;
  const int8_t* cg = codes + g * T * D + sub * 16;
  const float* sg = scales + g * T;
  const int64_t t0 = tile * (ITERS * kS128Step) + wave * (8 * kS128U) + slot;
  struct Batch {
    u32x4 c[kS128U];
    float s[kS128U];
  };
  // unconditional loads (tokens past T re-read token T - 1, not stored)
  auto load = [&](Batch& B, int it) {
#pragma unroll
    for (int u = 0; u < kS128U; ++u) {
      const int64_t t = std::min<int64_t>(t0 + it * (32 * kS128U) + u * 8, T - 1);
      B.c[u] = ld_stream(reinterpret_cast<const u32x4*>(cg + t * D));
      if constexpr (!CH) B.s[u] = sg[t];
    }
  };
  Batch ba, bb;
  load(ba, 0);
  const TQ* qg = q + g * NQ * D;
  for (int i = threadIdx.x; i < NQ * D; i += 256) {
    if constexpr (CH)
      qs[i] = to_f32(qg[i]) * scales[g * D + (i & (D - 1))];
    else
      qs[i] = to_f32(qg[i]);
  }
  __syncthreads();
  float qv[NQ][16];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4 x = reinterpret_cast<const f32x4*>(qs + j * D + sub * 16)[v];
      qv[j][4 * v] = x[0]; qv[j][4 * v + 1] = x[1]; qv[j][4 * v + 2] = x[2]; qv[j][4 * v + 3] = x[3];
    }
  auto score = [&](const Batch& B, int it) {
#pragma unroll
    for (int u = 0; u < kS128U; ++u) {
      const int64_t t = t0 + it * (32 * kS128U) + u * 8;
      float cf[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) cf[e] = i8_to_f32(B.c[u][e >> 2], e & 3);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) a = __builtin_fmaf(qv[j][e], cf[e], a);
        float tot = seg_sum_f32<8>(a);
        if constexpr (!CH) tot = tot * B.s[u];
        if (sub == 0 && t < T) scores[(g * NQ + j) * T + t] = tot;
      }
    }
  };
#pragma unroll
  for (int it = 0; it < ITERS; it += 2) {
    if (it + 1 < ITERS) load(bb, it + 1);
    score(ba, it);
    if (it + 2 < ITERS) load(ba, it + 2);
    if (it + 1 < ITERS) score(bb, it + 1);
  }
}

// Scale-folded INT8 score on the matrix cores, d = 128, several queries per
// group (grouped-query attention shares a head's codes among its queries):
// v_mfma_f32_16x16x32_f16 with 16 tokens' codes as the A operand (int8 ->
// binary16 is exact: bytes b ^ 0x80 placed under the exponent of 1024 by a
// byte permute, minus 1152 in one packed fp16 add) and the queries as the B
// operand's columns.  fp16 x int8 products are exact in binary32; the
// accumulation is binary32 (in the matrix core's order).  fp32 queries, and
// per-channel queries q_c s_c, are scaled per query by a power of two (max
// |v| into [2^14, 2^15)) and split into binary16 hi + lo (hi: the value with
// its 13 low significand bits cleared; lo: the remainder rounded toward
// zero, within 2^-20 relative of the scaled value): columns j and j + 8 of
// the same multiply, summed afterwards, then unscaled exactly.  A wave loads
// a 16-token tile as whole rows (each instruction reads 8 rows, 1 KiB
// contiguous: loading the A fragments directly would read 16 half-rows per
// instruction, measured 18 % slower) and reshapes it through its own 2 KiB
// of LDS; lane (n, kq) = (lane % 16, lane / 16) then holds channels
// 32 ks + 8 kq .. + 7 of token n at K-step ks, and the queries' fragments use
// the same channel order.  The result of token 4 kq + i, query column n is in
// accumulator i of lane (n, kq).
constexpr int kMfmaTiles = 4;                                   // 16-token tiles per wave pass
constexpr int kMfmaStep = 4 * 16 * kMfmaTiles;                  // tokens per block pass (4 waves)
constexpr int kMfmaMaxNq = 8;                                   // split query columns: 8 + 8
constexpr int64_t kMfmaMaxT = int64_t(1) << 23;                 // 32-bit token offsets

template <typename TQ, bool CH, int ITERS>
__global__ __launch_bounds__(256) void scores_int8_mfma_kernel(const TQ* __restrict__ q, int nq,
                                                               const int8_t* __restrict__ codes,
                                                               const float* __restrict__ scales,
                                                               int T, int64_t tiles,
                                                               float* __restrict__ scores) {
  constexpr int D = 128;
  constexpr bool SPLIT = CH || sizeof(TQ) == 4;
  __shared__ __align__(16) float qs[16 * D];
  __shared__ float qexp[16];
  // per wave: one 16-token tile of codes (2 KiB), row r at 128 r, its
  // 16-byte chunk c at 16 (c ^ ((r / 2) mod 8)): the row writes and the
  // fragment reads below each touch 64 different banks per 32 lanes
  __shared__ __align__(16) uint32_t tileb[4][16 * D / 4];
  const int64_t g = blockIdx.x / tiles;
  const int tile = (int)(blockIdx.x % tiles);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int kq = lane >> 4;
  // per-group bases; token offsets inside a group are 32-bit (T * 128 < 2^31)
  const int8_t* cg = codes + g * (int64_t)T * D + 16 * (lane & 7);
  const float* sg = scales + g * (int64_t)T;
  const int tw = tile * (ITERS * kMfmaStep) + wave * (16 * kMfmaTiles);
  struct Batch {
    u32x4 c[kMfmaTiles][2];
    float s;                                   // scale of token `lane` of the pass
  };
  // unconditional loads (tokens past T re-read token T - 1, not stored)
  auto load = [&](Batch& B, int it) {
    const int tb = tw + it * kMfmaStep;
#pragma unroll
    for (int u = 0; u < kMfmaTiles; ++u)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        // whole rows: 8 tokens x 128 B (1 KiB contiguous) per instruction
        const int tr = min(tb + 16 * u + 8 * a + (lane >> 3), T - 1);
        B.c[u][a] = ld_stream(reinterpret_cast<const u32x4*>(cg + tr * D));
      }
    if constexpr (!CH) B.s = sg[min(tb + lane, T - 1)];
  };
  Batch ba, bb;
  load(ba, 0);

  // queries (times the channel scales) in LDS as binary32, then each split
  // query's power-of-two exponent
  const TQ* qg = q + g * nq * D;
  for (int i = threadIdx.x; i < 16 * D; i += 256) {
    const int j = i / D, c = i % D;
    float v = 0.0f;
    if (j < nq) {
      v = to_f32(qg[j * D + c]);
      if constexpr (CH) v = v * scales[g * D + c];
    }
    qs[i] = v;
  }
  __syncthreads();
  if constexpr (SPLIT) {
    if (threadIdx.x < kMfmaMaxNq) {
      uint32_t mx = 0;
      for (int c = 0; c < D; ++c) mx = max(mx, abs_bits(qs[threadIdx.x * D + c]));
      // scale 2^(14 - e) with e the exponent of the largest magnitude
      const int e = mx == 0 ? 0 : (int)((mx >> 23) & 0xFF) - 127;
      qexp[threadIdx.x] = __builtin_ldexpf(1.0f, min(14 - e, 126));
    }
    __syncthreads();
  }
  // B fragments: column n, K-step ks, element e = channel 32 ks + 8 kq + e
  f16x8 bq[4];
  {
    const int j = SPLIT ? (n & 7) : n;
    const bool lo = SPLIT && n >= 8;
    const float sc = SPLIT ? qexp[j] : 1.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = qs[j * D + 32 * ks + 8 * kq + e] * sc;
        if constexpr (SPLIT) {
          const float hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xFFFFE000u);
          const auto pk = __builtin_amdgcn_cvt_pkrtz(lo ? v - hi : hi, 0.0f);
          bq[ks][e] = pk[0];
        } else {
          bq[ks][e] = (_Float16)v;
        }
      }
  }
  float unscale = 1.0f;
  if constexpr (SPLIT) unscale = 1.0f / qexp[n & 7];      // exact: a power of two
  const int jq = SPLIT ? (n & 7) : n;                     // query of this lane's column
  const bool writer = SPLIT ? (n < 8 && n < nq) : (n < nq);
  float* og = scores + (g * nq + (writer ? jq : 0)) * (int64_t)T;
  // whole 16-byte runs of 4 tokens when every query row starts 16-byte aligned
  const bool vec_out = (T & 3) == 0;

  // 8 codes (two words) -> 8 binary16 values
  auto codes_f16 = [](uint32_t w0, uint32_t w1) {
    const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
    f16x8 r;
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    uint32_t p[4];
    p[0] = __builtin_amdgcn_perm(0x64646464u, x0, 0x07010700u);   // bytes: b0, 0x64, b1, 0x64
    p[1] = __builtin_amdgcn_perm(0x64646464u, x0, 0x07030702u);
    p[2] = __builtin_amdgcn_perm(0x64646464u, x1, 0x07010700u);
    p[3] = __builtin_amdgcn_perm(0x64646464u, x1, 0x07030702u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const h2 v = __builtin_bit_cast(h2, p[i]) + bias;
      r[2 * i] = v[0];
      r[2 * i + 1] = v[1];
    }
    return r;
  };
  uint32_t* tl = tileb[wave];
  // this lane's row writes (row 8 a + lane / 8, chunk lane % 8) and fragment
  // reads (row n, bytes [32 ks + 8 kq, + 8)), as dword offsets
  uint32_t woff[2], roff[4];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int r = 8 * a + (lane >> 3);
    woff[a] = 32 * r + 4 * ((lane & 7) ^ ((r >> 1) & 7));
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int c = 2 * ks + (kq >> 1);
    roff[ks] = 32 * n + 4 * (c ^ ((n >> 1) & 7)) + 2 * (kq & 1);
  }
  auto score = [&](const Batch& B, int it) {
    const int tb = tw + it * kMfmaStep;
#pragma unroll
    for (int u = 0; u < kMfmaTiles; ++u) {
      // rows -> LDS -> A fragments (the wave's own tile; LDS operations of
      // one wave complete in order, the asm statements keep the compiler
      // from moving the reads above the writes or the next writes above
      // the reads)
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int a = 0; a < 2; ++a) *reinterpret_cast<u32x4*>(tl + woff[a]) = B.c[u][a];
      __asm__ volatile("" ::: "memory");
      u32x2 cw[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) cw[ks] = *reinterpret_cast<const u32x2*>(tl + roff[ks]);
      __asm__ volatile("" ::: "memory");
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f16x8 a = codes_f16(cw[ks][0], cw[ks][1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bq[ks], acc, 0, 0, 0);
      }
      const int t0 = tb + 16 * u + 4 * kq;
      f32x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[i];
        if constexpr (SPLIT) {
          // the lo column's partial sum (lane n + 8) added to the hi one
          v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x201F));
          v *= unscale;
        }
        if constexpr (!CH) {
          // token 16 u + 4 kq + i's scale from the lane that loaded it
          v *= __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((16 * u + 4 * kq + i) << 2,
                                                                      __builtin_bit_cast(int, B.s)));
        }
        out[i] = v;
      }
      if (writer) {
        if (vec_out && t0 + 3 < T) {
          *reinterpret_cast<f32x4*>(og + t0) = out;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + i < T) og[t0 + i] = out[i];
        }
      }
    }
  };
#pragma unroll
  for (int it = 0; it < ITERS; it += 2) {
    if (it + 1 < ITERS) load(bb, it + 1);
    score(ba, it);
    if (it + 2 < ITERS) load(ba, it + 2);
    if (it + 1 < ITERS) score(bb, it + 1);
  }
}

template <typename TQ, bool CH, int ITERS>
static hipError_t scores_mfma_launch_it(const TQ* q, int64_t groups, int nq, const int8_t* codes,
                                        const float* scales, int64_t T, float* scores,
                                        hipStream_t s) {
  const int64_t tiles = (T + ITERS * kMfmaStep - 1) / (ITERS * kMfmaStep);
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / tiles);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    hipLaunchKernelGGL((scores_int8_mfma_kernel<TQ, CH, ITERS>), dim3((unsigned)(ng * tiles)),
                       dim3(256), 0, s, q + g0 * nq * 128, nq, codes + g0 * T * 128,
                       scales + g0 * (CH ? 128 : T), (int)T, tiles, scores + g0 * nq * T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TQ, bool CH>
static hipError_t scores_mfma_launch(const TQ* q, int64_t groups, int nq, const int8_t* codes,
                                     const float* scales, int64_t T, float* scores,
                                     hipStream_t s) {
  const int64_t rows = groups * T;
  if (rows >= 1024LL * 4 * kMfmaStep)
    return scores_mfma_launch_it<TQ, CH, 4>(q, groups, nq, codes, scales, T, scores, s);
  return scores_mfma_launch_it<TQ, CH, 1>(q, groups, nq, codes, scales, T, scores, s);
}

template <typename TQ, bool CH, int ITERS>
static hipError_t scores_d128_launch_it(const TQ* q, int64_t groups, int nq, const int8_t* codes,
                                        const float* scales, int64_t T, float* scores,
                                        hipStream_t s) {
  const int64_t tiles = (T + ITERS * kS128Step - 1) / (ITERS * kS128Step);
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / tiles);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    const TQ* qp = q + g0 * nq * 128;
    const int8_t* cp = codes + g0 * T * 128;
    const float* sp = scales + g0 * (CH ? 128 : T);
    float* op = scores + g0 * nq * T;
    const dim3 grid((unsigned)(ng * tiles));
    switch (nq) {
      case 1: hipLaunchKernelGGL((scores_int8_d128_kernel<TQ, 1, CH, ITERS>), grid, dim3(256), 0, s, qp, cp, sp, T, tiles, op); break;
      case 2: hipLaunchKernelGGL((scores_int8_d128_kernel<TQ, 2, CH, ITERS>), grid, dim3(256), 0, s, qp, cp, sp, T, tiles, op); break;
      case 3: hipLaunchKernelGGL((scores_int8_d128_kernel<TQ, 3, CH, ITERS>), grid, dim3(256), 0, s, qp, cp, sp, T, tiles, op); break;
      default: hipLaunchKernelGGL((scores_int8_d128_kernel<TQ, 4, CH, ITERS>), grid, dim3(256), 0, s, qp, cp, sp, T, tiles, op); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Longer token ranges per block where the grid stays at >= 1024 blocks
// (4 per compute unit).
template <typename TQ, bool CH>
static hipError_t scores_d128_launch(const TQ* q, int64_t groups, int nq, const int8_t* codes,
                                     const float* scales, int64_t T, float* scores,
                                     hipStream_t s) {
  const int64_t rows = groups * T;
  // several queries: 8 iterations per block on long caches; one query: at
  // most 2 (at 32 x 262144 tokens, 186 us against 197 us with 8, while 4
  // queries take 252 us with 8 and 294 us with 2)
  if (nq > 1 && rows >= 1024LL * 8 * kS128Step)
    return scores_d128_launch_it<TQ, CH, 8>(q, groups, nq, codes, scales, T, scores, s);
  if (rows >= 1024LL * 2 * kS128Step)
    return scores_d128_launch_it<TQ, CH, 2>(q, groups, nq, codes, scales, T, scores, s);
  return scores_d128_launch_it<TQ, CH, 1>(q, groups, nq, codes, scales, T, scores, s);
}

template <typename TQ>
static hipError_t scores_dispatch(const TQ* q, int64_t groups, int nq, const int8_t* codes,
                                  const float* scales, int64_t T, int d, float* scores,
                                  hipStream_t s) {
  // Two or three queries over fewer than 2^20 rows: the vector path's shorter start-up beats
  // the matrix-core tile (5.6 vs 6.5 us at 32 x 4096); from four queries on, or on larger
  // caches, the matrix cores are as fast or faster.
  const bool small_few = nq <= 3 && groups * T < (int64_t(1) << 20);
  if (d == 128 && nq >= 2 && nq <= (sizeof(TQ) == 2 ? 16 : kMfmaMaxNq) && T <= kMfmaMaxT &&
      !small_few)
    return scores_mfma_launch<TQ, false>(q, groups, nq, codes, scales, T, scores, s);
  if (d == 128 && nq <= 4) return scores_d128_launch<TQ, false>(q, groups, nq, codes, scales, T, scores, s);
  const int64_t tiles = (T + kScoreTokensPerBlock - 1) / kScoreTokensPerBlock;
  // launch in slices of whole groups so grid.x stays far below 2^32
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / tiles);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    const TQ* qp = q + g0 * nq * d;
    const int8_t* cp = codes + g0 * T * d;
    const float* sp = scales + g0 * T;
    float* op = scores + g0 * nq * T;
    if (d <= kScoreLdsFloats)
      hipLaunchKernelGGL((scores_int8_kernel<TQ, true>), dim3((unsigned)(ng * tiles)), dim3(256), 0,
                         s, qp, nq, cp, sp, T, d, tiles, op);
    else
      hipLaunchKernelGGL((scores_int8_kernel<TQ, false>), dim3((unsigned)(ng * tiles)), dim3(256),
                         0, s, qp, nq, cp, sp, T, d, tiles, op);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TQ>
static hipError_t scores_channel_dispatch(const TQ* q, int64_t groups, int nq, const int8_t* codes,
                                          const float* scales, int64_t T, int d, float* scores,
                                          hipStream_t s) {
  if (d == 128 && nq >= 2 && nq <= kMfmaMaxNq && T <= kMfmaMaxT)
    return scores_mfma_launch<TQ, true>(q, groups, nq, codes, scales, T, scores, s);
  if (d == 128 && nq <= 4) return scores_d128_launch<TQ, true>(q, groups, nq, codes, scales, T, scores, s);
  const int64_t tiles = (T + kScoreTokensPerBlock - 1) / kScoreTokensPerBlock;
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / tiles);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    hipLaunchKernelGGL((scores_int8_kernel<TQ, true, true>), dim3((unsigned)(ng * tiles)),
                       dim3(256), 0, s, q + g0 * nq * d, nq, codes + g0 * T * d, scales + g0 * d,
                       T, d, tiles, scores + g0 * nq * T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_scores_int8_channel(const void* q, int q_f16, int64_t groups, int nq,
                                      const int8_t* codes, const float* scales, int64_t T, int d,
                                      float* scores, hipStream_t s) {
  if (q_f16)
    return scores_channel_dispatch(static_cast<const _Float16*>(q), groups, nq, codes, scales, T,
                                   d, scores, s);
  return scores_channel_dispatch(static_cast<const float*>(q), groups, nq, codes, scales, T, d,
                                 scores, s);
}

hipError_t launch_scores_int8(const void* q, int q_f16, int64_t groups, int nq,
                              const int8_t* codes, const float* scales, int64_t T, int d,
                              float* scores, hipStream_t s) {
  if (q_f16)
    return scores_dispatch(static_cast<const _Float16*>(q), groups, nq, codes, scales, T, d,
                           scores, s);
  return scores_dispatch(static_cast<const float*>(q), groups, nq, codes, scales, T, d, scores, s);
}

}  // namespace kvq
