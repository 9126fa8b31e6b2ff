// QJL on the residual of the INT4 quantizer: two-stage key compression and
// its score, for gfx950.
//
// Method: the TurboQuant news item (after ArsTechnica) compresses in two
// stages, a scalar first stage whose residual error a 1-bit QJL layer then
// corrects, for a more accurate attention-score estimate; QJL (arXiv
// 2406.03482, abstract) gives the sign sketch and the asymmetric estimator;
// the first stage here is the asymmetric group-wise INT4 formula of the
// Q-TensorFormer model card (section 6).  Per key row k:
//   codes, step s, offset z per group      (as kvq_quantize_int4)
//   k_hat = RN32(RN32(c * s) + z),  r = RN32(k - k_hat)
//   bits = [S r >= 0] (LSB-first words),  n = RN16(||r||)
// and per query q (y = S q):
//   sigma = q . k_hat + sqrt(pi/2) / m * n * sum_i (2 b_i - 1) y_i.
//
// Sketch, fp16 keys and S, d = 128, m = 256: one fused pass.  A wave holds
// 32 tokens as the B operand of v_mfma_f32_32x32x16_f16 (lane = token j,
// half h: channels 16 ks + 8 h .. + 8), so a token's groups are reduced with
// one v_permlane32_swap per min and max; the residual (binary32) is scaled
// per token by a power of two (max |r| into [2^14, 2^15)) and split into two
// binary16 parts hi + lo (hi: the value's top 11 significand bits, lo: the
// exact remainder, rounded toward zero), which carry it to within 2^-20
// relative; S r is accumulated from both parts on the matrix cores (S
// fragments resident in LDS, as in the plain sketch).  Other shapes: the INT4 quantizer, then one
// thread per (row, sign word) with binary32 dot products.
#include "kvq_device.h"
#include "kvq_int4_device.h"
#include "kvq_launch.h"
#include "kvq_qjl_device.h"

#include <algorithm>

namespace kvq {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kResThreads = 512;
constexpr int kResWaves = kResThreads / 64;
constexpr int kResKS = 8;   // d = 128: 8 K-steps of 16 channels
constexpr int kResMT = 8;   // m = 256: 8 projection tiles of 32
constexpr int kResRing = 2; // token tiles in flight per wave

// Sign word from a projection tile's accumulators: bit = [P >= 0], assembled
// as in the plain sketch (accumulator r of lane (j, h) holds projection
// 32 mt + 16 h + r; the halves' 16 bits are exchanged).
__device__ __forceinline__ uint32_t res_acc_word(const f32x16& acc) {
  uint32_t sb = 0;
#pragma unroll
  for (int r = 15; r >= 0; --r) {
    const float pr = acc[r];
    sb = __builtin_amdgcn_alignbit(sb, __builtin_bit_cast(uint32_t, pr), 31);
  }
  uint32_t lo, hi;
  halves_u32(~sb & 0xFFFFu, lo, hi);
  return lo | (hi << 16);
}

// codes_rcp for t = RN32(x - z) given, without the clamp: t >= 0 and
// t / s <= 15 + 2^-19, so the rounded quotient is already in [0, 15].
__device__ __forceinline__ void codes_rcp_t(const float (&t)[8], float sdiv, float r,
                                            bool divide, float (&c)[8]) {
  bool near = divide;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = t[e] * r;
    c[e] = __builtin_rintf(q);
    near |= __builtin_fabsf(q - c[e]) > 0.5f - 0x1p-16f;
  }
  if (near) {
    __asm__ volatile("");
#pragma unroll
    for (int e = 0; e < 8; ++e) c[e] = __builtin_rintf(t[e] / sdiv);
  }
}

__device__ __forceinline__ float other_half_f32(float v, bool take_hi) {
  uint32_t lo, hi;
  halves_u32(__builtin_bit_cast(uint32_t, v), lo, hi);
  return __builtin_bit_cast(float, take_hi ? hi : lo);
}

// Fused INT4 + residual sketch for fp16 keys, fp16 S, d = 128, m = 256 and
// group size G in {16, 32, 64, 128}.  Persistent grid; each wave strides
// over 32-token tiles with a ring of kResRing tiles in flight (loads
// unconditional, clamped to the last row past the end; nothing of those
// tokens is stored).
template <int G>
__global__ __launch_bounds__(kResThreads) __attribute__((amdgpu_waves_per_eu(2)))
void residual_sketch_kernel(const _Float16* __restrict__ k, int64_t rows,
                            const _Float16* __restrict__ S, uint8_t* __restrict__ codes,
                            float* __restrict__ steps, float* __restrict__ offsets,
                            uint32_t* __restrict__ bits, uint16_t* __restrict__ norms) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  f16x8* sfrag = reinterpret_cast<f16x8*>(lds_raw);
  constexpr int D = kResKS * 16;
  constexpr int NG = D / G;          // groups per row
  constexpr int KPG = G / 16;        // K-steps per group (G >= 16)
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  // S -> LDS in fragment order (as the plain sketch): fragment (mt, ks),
  // lane l holds S[32 mt + perm(l % 32)][16 ks + 8 (l / 32) .. + 8].
  for (int idx = tid; idx < kResMT * kResKS * 64; idx += kResThreads) {
    const int l = idx & 63;
    const int frag = idx >> 6;
    const int mt = frag / kResKS, ks = frag % kResKS;
    const int srow = 32 * mt + sketch_row_perm(l & 31);
    sfrag[idx] = *reinterpret_cast<const f16x8*>(S + (int64_t)srow * D + 16 * ks + 8 * (l >> 5));
  }
  __syncthreads();

  const int64_t tiles = (rows + 31) / 32;
  auto load = [&](f16x8 (&b)[kResKS], int64_t tile) {
    const int64_t tok = std::min<int64_t>(tile * 32 + col, rows - 1);
    const _Float16* kr = k + tok * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kResKS; ++ks) b[ks] = ld_stream(reinterpret_cast<const f16x8*>(kr + 16 * ks));
  };

  auto process = [&](const f16x8 (&b)[kResKS], int64_t tile) {
    const int64_t tok = tile * 32 + col;
    int off = 0;
    asm volatile("" : "+v"(off));
    const f16x8* sf = sfrag + off;

    // 1) group min / max: this lane's 8 channels per K-step, then the other
    //    half's
    float mn[NG], mx[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      // packed binary16 min / max (exact), two values per instruction
      f16x2 pmn = {b[j * KPG][0], b[j * KPG][1]}, pmx = pmn;
#pragma unroll
      for (int kk = 0; kk < KPG; ++kk)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const f16x2 v2 = {b[j * KPG + kk][e], b[j * KPG + kk][e + 1]};
          pmn = __builtin_elementwise_min(pmn, v2);
          pmx = __builtin_elementwise_max(pmx, v2);
        }
      mn[j] = __builtin_fminf((float)pmn[0], (float)pmn[1]);
      mx[j] = __builtin_fmaxf((float)pmx[0], (float)pmx[1]);
      mn[j] = __builtin_fminf(mn[j], other_half_f32(mn[j], h == 0));
      mx[j] = __builtin_fmaxf(mx[j], other_half_f32(mx[j], h == 0));
    }
    float st[NG], sdiv[NG], rc[NG];
    bool dv[NG];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      st[j] = group_step(mn[j], mx[j]);
      sdiv[j] = step_divisor(st[j]);
      rc[j] = __builtin_amdgcn_rcpf(sdiv[j]);
      dv[j] = !rcp_ok(sdiv[j]);
    }

    // the encode runs at raised wave priority, the multiplies at the base
    // one: the other wave of the SIMD then issues its MFMAs while this one
    // is in its vector-ALU phase (368 -> 348 us at 8 x 32 x 8192 x 128)
    __builtin_amdgcn_s_setprio(1);
    // 2) codes, reconstruction and residual
    uint32_t cw[kResKS];
    float rr[kResKS][8];
    float ss = 0.0f, am = 0.0f;
#pragma unroll
    for (int ks = 0; ks < kResKS; ++ks) {
      const int j = ks / KPG;
      float tv[8], c[8];
      // t = RN32(x - z) straight from the binary16 key (a mixed-precision
      // fused multiply-add by 1 rounds once)
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e] = __builtin_fmaf((float)b[ks][e], 1.0f, -mn[j]);
      codes_rcp_t(tv, sdiv[j], rc[j], dv[j], c);
      // codes to bytes (exact integers, so the conversion's rounding is
      // moot), even elements in one word and odd in another, then nibbles
      uint32_t ev = 0, od = 0;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        ev = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * e2], e2, ev);
        od = __builtin_amdgcn_cvt_pk_u8_f32(c[2 * e2 + 1], e2, od);
      }
      cw[ks] = ev | (od << 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        rr[ks][e] = __builtin_fmaf((float)b[ks][e], 1.0f, -recon4(c[e], st[j], mn[j]));
        ss = __builtin_fmaf(rr[ks][e], rr[ks][e], ss);
        am = __builtin_fmaxf(am, __builtin_fabsf(rr[ks][e]));
      }
    }
    ss = ss + other_half_f32(ss, h == 0);
    am = __builtin_fmaxf(am, other_half_f32(am, h == 0));

    // 3) residual scaled by 2^(15 - e) (am = f 2^e, f in [0.5, 1)) and split
    //    into binary16 hi + lo
    // hi = v with its 13 low significand bits cleared (binary16-representable
    // for |v| >= 2^-14), lo = v - hi exactly; both converted toward zero
    // two at a time (lo's truncation is below 2^-20 |v|)
    const int sc = 15 - __builtin_amdgcn_frexp_expf(am);
    f16x8 bh[kResKS], bl[kResKS];
#pragma unroll
    for (int ks = 0; ks < kResKS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float v0 = __builtin_amdgcn_ldexpf(rr[ks][e], sc);
        const float v1 = __builtin_amdgcn_ldexpf(rr[ks][e + 1], sc);
        const float h0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v0) & 0xFFFFE000u);
        const float h1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v1) & 0xFFFFE000u);
        const auto ph = __builtin_amdgcn_cvt_pkrtz(h0, h1);
        const auto pl = __builtin_amdgcn_cvt_pkrtz(v0 - h0, v1 - h1);
        bh[ks][e] = ph[0]; bh[ks][e + 1] = ph[1];
        bl[ks][e] = pl[0]; bl[ks][e + 1] = pl[1];
      }

    // 4) sign words
    uint32_t wbuf[kResMT];
    // one accumulator chain per projection tile (hi and lo parts in turn);
    // the sign word of tile mt - 1 is taken between the MFMAs of tile mt
    f32x16 accA, accB;
    auto chain = [&](int mt, f32x16& acc) {
      acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < kResKS; ++ks) {
        const f16x8 a = sf[(mt * kResKS + ks) * 64 + lane];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bl[ks], acc, 0, 0, 0);
      }
    };
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    chain(0, accA);
#pragma unroll
    for (int mt = 1; mt <= kResMT; ++mt) {
      __builtin_amdgcn_sched_barrier(0);
      uint32_t w;
      if (mt & 1) {
        if (mt < kResMT) chain(mt, accB);
        w = res_acc_word(accA);
      } else {
        if (mt < kResMT) chain(mt, accA);
        w = res_acc_word(accB);
      }
      if (mt < kResMT) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // LDS reads
#pragma unroll
        for (int ks = 0; ks < kResKS; ++ks) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMA
          if (ks + 2 < kResKS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);      // VALU
        }
      }
      wbuf[mt - 1] = w;
    }

    // 5) stores: half h writes code bytes [32 h, 32 h + 32), the steps
    //    (h = 0) or the offsets (h = 1), sign words [4 h, 4 h + 4) and, for
    //    h = 0, the norm.  Lane-mask blends rather than selects, which the
    //    compiler would turn into dynamically indexed (scratch) arrays.
    uint32_t clo[kResKS], chi[kResKS];
#pragma unroll
    for (int ks = 0; ks < kResKS; ++ks) halves_u32(cw[ks], clo[ks], chi[ks]);
    if (tok < rows) {
      const uint32_t m0 = h == 0 ? 0xFFFFFFFFu : 0u;
      u32x4 cv[2];
#pragma unroll
      for (int q4 = 0; q4 < 2; ++q4)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int idx = 4 * q4 + jj;       // word of this half's 8
          const int ks0 = idx / 2, ks1 = 4 + idx / 2;
          const uint32_t a = (idx & 1) ? chi[ks0] : clo[ks0];
          const uint32_t bb = (idx & 1) ? chi[ks1] : clo[ks1];
          cv[q4][jj] = (a & m0) | (bb & ~m0);
        }
      u32x4* cdst = reinterpret_cast<u32x4*>(codes + tok * (D / 2) + 32 * h);
      cdst[0] = cv[0];
      cdst[1] = cv[1];
      float* sz = (h == 0 ? steps : offsets) + tok * NG;
#pragma unroll
      for (int j = 0; j < NG; ++j)
        sz[j] = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, st[j]) & m0) |
                                              (__builtin_bit_cast(uint32_t, mn[j]) & ~m0));
      u32x4 wv;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) wv[jj] = (wbuf[jj] & m0) | (wbuf[4 + jj] & ~m0);
      *reinterpret_cast<u32x4*>(bits + tok * kResMT + 4 * h) = wv;
      if (h == 0) norms[tok] = f32_to_f16_bits(__builtin_sqrtf(ss));
    }
  };

  const int64_t stride = (int64_t)gridDim.x * kResWaves;
  const int64_t first = (int64_t)blockIdx.x * kResWaves + wave;
  if (first >= tiles) return;
  f16x8 bq[kResRing][kResKS];
#pragma unroll
  for (int r = 0; r < kResRing; ++r) load(bq[r], std::min(first + r * stride, tiles - 1));
  for (int64_t t0 = first;; t0 += kResRing * stride) {
#pragma unroll
    for (int r = 0; r < kResRing; ++r) {
      const int64_t t = t0 + r * stride;
      process(bq[r], t);
      if (t + stride >= tiles) return;
      load(bq[r], std::min(t + kResRing * stride, tiles - 1));
    }
  }
}

// Residual value j of a row, from the key and its stored INT4 encoding.
template <typename TK>
__device__ __forceinline__ float residual_at(const TK* kr, const uint8_t* cr, const float* sr,
                                             const float* zr, int g, int j) {
  const uint32_t c = (cr[j >> 1] >> (4 * (j & 1))) & 0xFu;
  const int grp = j / g;
  return to_f32(kr[j]) - recon4((float)c, sr[grp], zr[grp]);
}

// Residual sketch, any shape: one thread per (row, sign word), binary32 dot
// products of S rows with the residual (rebuilt from the key and the codes
// the quantizer wrote); the word-0 thread also writes the norm.
template <typename TK, typename TS>
__global__ __launch_bounds__(256) void residual_sketch_generic_kernel(
    const TK* __restrict__ k, int64_t rows, int d, int g, const TS* __restrict__ S, int m,
    const uint8_t* __restrict__ codes, const float* __restrict__ steps,
    const float* __restrict__ offsets, uint32_t* __restrict__ bits, uint16_t* __restrict__ norms) {
  const int words = m / 32;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / words;
  const int w = (int)(gid % words);
  if (row >= rows) return;
  const TK* kr = k + row * d;
  const uint8_t* cr = codes + row * (d / 2);
  const float* sr = steps + row * (d / g);
  const float* zr = offsets + row * (d / g);
  uint32_t word = 0;
  for (int i = 0; i < 32; ++i) {
    const TS* srow = S + (int64_t)(32 * w + i) * d;
    float p = 0.0f;
    for (int j = 0; j < d; ++j) p = __builtin_fmaf(to_f32(srow[j]), residual_at(kr, cr, sr, zr, g, j), p);
    word |= (p >= 0.0f ? 1u : 0u) << i;
  }
  bits[row * words + w] = word;
  if (w == 0) {
    float acc = 0.0f;
    for (int j = 0; j < d; ++j) {
      const float v = residual_at(kr, cr, sr, zr, g, j);
      acc = __builtin_fmaf(v, v, acc);
    }
    norms[row] = f32_to_f16_bits(__builtin_sqrtf(acc));
  }
}

template <int G>
static hipError_t residual_sketch_launch(const _Float16* k, int64_t rows, const _Float16* S,
                                         uint8_t* codes, float* steps, float* offsets,
                                         uint32_t* bits, uint16_t* norms, const DeviceInfo& dev,
                                         hipStream_t st) {
  const size_t lds = (size_t)kResMT * 32 * kResKS * 16 * sizeof(_Float16);   // 64 KiB
  const int64_t tiles = (rows + 31) / 32;
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, residual_sketch_kernel<G>,
                                                              kResThreads, lds);
  if (e != hipSuccess) return e;
  const int64_t want = (tiles + kResWaves - 1) / kResWaves;
  const int64_t cap = (int64_t)dev.cus * std::max(1, per_cu);
  const int64_t blocks = std::max<int64_t>(1, std::min(want, cap));
  hipLaunchKernelGGL(residual_sketch_kernel<G>, dim3((unsigned)blocks), dim3(kResThreads), lds, st,
                     k, rows, S, codes, steps, offsets, bits, norms);
  return hipGetLastError();
}

template <typename TK, typename TS>
static hipError_t residual_sketch_generic(const TK* k, int64_t rows, int d, int g, const TS* S,
                                          int m, const uint8_t* codes, const float* steps,
                                          const float* offsets, uint32_t* bits, uint16_t* norms,
                                          hipStream_t st) {
  const int words = m / 32;
  const int64_t rows_per = std::max<int64_t>(1, (int64_t(1) << 30) / words);
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per) {
    const int64_t nr = std::min(rows_per, rows - r0);
    const int64_t nb = (nr * words + 255) / 256;
    hipLaunchKernelGGL((residual_sketch_generic_kernel<TK, TS>), dim3((unsigned)nb), dim3(256), 0,
                       st, k + r0 * d, nr, d, g, S, m, codes + r0 * (d / 2), steps + r0 * (d / g),
                       offsets + r0 * (d / g), bits + r0 * words, norms + r0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_residual_sketch(const void* k, int k_f16, int64_t rows, int d, int g,
                                  const void* S, int S_f16, int m, uint8_t* codes, float* steps,
                                  float* offsets, uint32_t* bits, uint16_t* norms,
                                  const DeviceInfo& dev, hipStream_t st) {
  if (k_f16 && S_f16 && d == 128 && m == 256 && dev.lds_per_block >= 64 * 1024) {
    const _Float16* kh = static_cast<const _Float16*>(k);
    const _Float16* Sh = static_cast<const _Float16*>(S);
    switch (g) {
      case 16: return residual_sketch_launch<16>(kh, rows, Sh, codes, steps, offsets, bits, norms, dev, st);
      case 32: return residual_sketch_launch<32>(kh, rows, Sh, codes, steps, offsets, bits, norms, dev, st);
      case 64: return residual_sketch_launch<64>(kh, rows, Sh, codes, steps, offsets, bits, norms, dev, st);
      case 128: return residual_sketch_launch<128>(kh, rows, Sh, codes, steps, offsets, bits, norms, dev, st);
      default: break;
    }
  }
  hipError_t e = launch_quantize_int4(k, k_f16, rows, d, g, codes, steps, offsets, st);
  if (e != hipSuccess) return e;
  if (k_f16) {
    const _Float16* kh = static_cast<const _Float16*>(k);
    if (S_f16)
      return residual_sketch_generic(kh, rows, d, g, static_cast<const _Float16*>(S), m, codes,
                                     steps, offsets, bits, norms, st);
    return residual_sketch_generic(kh, rows, d, g, static_cast<const float*>(S), m, codes, steps,
                                   offsets, bits, norms, st);
  }
  const float* kf = static_cast<const float*>(k);
  if (S_f16)
    return residual_sketch_generic(kf, rows, d, g, static_cast<const _Float16*>(S), m, codes, steps,
                                   offsets, bits, norms, st);
  return residual_sketch_generic(kf, rows, d, g, static_cast<const float*>(S), m, codes, steps,
                                 offsets, bits, norms, st);
}


// ---------------------------------------------------------------------------
// Scores.  fp16 S, d = 128, m = 256: one workgroup per (group, query, tile of
// kRsTile tokens); 4 lanes per token, lane `sub` holding channels
// 32 sub .. 32 sub + 31 of the query in registers (binary32) and reading the
// token's codes for them (16 bytes), the steps and offsets of their groups,
// and sign words 2 sub, 2 sub + 1.  The INT4 part is folded per group,
// s * sum_i q_i c_i + z * sum_i q_i (sums over the lane's channels of the
// group); the QJL part is 8 lookups of byte tables T_p[v] = sum_{j<8}
// (bit j of v ? +1 : -1) y_{8p+j}, stored as 256 rows v of the 32 tables'
// entries.  Lane (token slot tt, sub) reads table 8 sub + ((b + tt) mod 8) at
// step b, so the 32 lanes of a half-wave read 32 different tables, i.e. 32
// different LDS banks, whatever the bytes; the lane's 8 sign bytes are
// rotated by tt mod 8 beforehand.  The quad's 4 partial scores are summed
// with DPP.
constexpr int kRsThreads = 256;
constexpr int kRsU = 4;                          // tokens in flight per lane
constexpr int kRsIters = 8;
constexpr int kRsTile = 64 * kRsU * kRsIters;    // 2048 tokens per workgroup
constexpr int kRsRowFloats = 32;
// 32 KiB, at LDS address 0: the lookups use the byte permute's result as the
// address itself, so the scores kernel declares no static __shared__ data
// (its dynamic LDS then starts at address 0)
constexpr int kRsLutFloats = 256 * kRsRowFloats;

// Tables of y[0..255] in rows of 32 entries: lut[32 v + p] = T_p[v] (same
// binary32 values as the other table builders: low-nibble partial sums plus
// a high-nibble sum).
__device__ void build_tables32(const float* y, float* lut) {
  for (int task = threadIdx.x; task < 32 * 16; task += blockDim.x) {
    const int p = task & 31;
    const int a = task >> 5;
    const float* yp = y + 8 * p;
    float lo[16];
    lo[0] = -(((yp[0] + yp[1]) + yp[2]) + yp[3]);
#pragma unroll
    for (int b = 1; b < 16; ++b) {
      const int low = b & (-b);
      const int j = __builtin_ctz(low);
      lo[b] = lo[b ^ low] + 2.0f * yp[j];
    }
    float hi = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) hi += ((a >> j) & 1) ? yp[4 + j] : -yp[4 + j];
#pragma unroll
    for (int b = 0; b < 16; ++b) lut[(16 * a + b) * kRsRowFloats + p] = hi + lo[b];
  }
}

// One lane's share of one token: code bytes of its 32 channels, its two sign
// words, the steps and offsets of the (one or two) groups its channels touch,
// the norm bits.
template <int GPL>
struct RsTok {
  u32x4 c;
  uint32_t w[2];
  float s[GPL], z[GPL];
  uint32_t n;
};

template <typename TQ, int G>
__global__ __launch_bounds__(kRsThreads) void scores_residual_kernel(
    const TQ* __restrict__ q, int nq, const _Float16* __restrict__ S,
    const uint8_t* __restrict__ codes, const float* __restrict__ steps,
    const float* __restrict__ offsets, const uint32_t* __restrict__ bits,
    const uint16_t* __restrict__ norms, int64_t T, int64_t tiles, float* __restrict__ scores) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  float* lut = reinterpret_cast<float*>(lds_raw);
  float* y = lut + kRsLutFloats;
  float* qs = y + 256;
  constexpr int D = 128, M = 256, NG = D / G;
  constexpr int GPL = G >= 32 ? 1 : 2;
  const int64_t gq = blockIdx.x / tiles;
  const int64_t tile = blockIdx.x % tiles;
  const int64_t grp = gq / nq;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int sub = lane & 3;
  const int tt = lane >> 2;
  const int j0 = (32 * sub) / G;                  // first group of the lane's channels
  const int64_t tb = tile * kRsTile + wave * 16 + tt;
  const uint8_t* cg = codes + grp * T * (D / 2);
  const float* sg = steps + grp * T * NG;
  const float* zg = offsets + grp * T * NG;
  const uint32_t* bg = bits + grp * T * (M / 32);
  const uint16_t* ngp = norms + grp * T;

  // loads are unconditional (tokens past T re-read token T - 1; their scores
  // are not stored)
  auto load = [&](RsTok<GPL> (&tk)[kRsU], int it) {
#pragma unroll
    for (int u = 0; u < kRsU; ++u) {
      const int64_t t = std::min<int64_t>(tb + 64 * (it * kRsU + u), T - 1);
      tk[u].c = ld_stream(reinterpret_cast<const u32x4*>(cg + t * (D / 2) + 16 * sub));
      const u32x2 wv = ld_stream(reinterpret_cast<const u32x2*>(bg + t * (M / 32) + 2 * sub));
      tk[u].w[0] = wv[0];
      tk[u].w[1] = wv[1];
#pragma unroll
      for (int k = 0; k < GPL; ++k) {
        tk[u].s[k] = sg[t * NG + j0 + k];
        tk[u].z[k] = zg[t * NG + j0 + k];
      }
      tk[u].n = ngp[t];
    }
  };

  // the S rows and the query arrive before any token is requested: a CU's
  // vector loads return in issue order, so rows queued behind token loads
  // (this wave's or the CU's other waves') would wait for HBM
  QueryProj16<TQ> pj;
  pj.issue(S, q + gq * D, M, D);
#pragma unroll
  for (int it = 0; it < 16; ++it) asm volatile("" ::"v"(pj.raw[it]));
  asm volatile("" ::"v"(pj.qreg));
  __builtin_amdgcn_sched_barrier(0);
  RsTok<GPL> ka[kRsU];
  load(ka, 0);
  __builtin_amdgcn_sched_barrier(0);
  pj.finish(qs, y, M, D);
  __syncthreads();
  build_tables32(y, lut);
  // the lane's query channels (binary32) in nibble order, and their sums per
  // group
  float qv[32];
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const f32x4 x = reinterpret_cast<const f32x4*>(qs + 32 * sub)[v];
    qv[4 * v] = x[0]; qv[4 * v + 1] = x[1]; qv[4 * v + 2] = x[2]; qv[4 * v + 3] = x[3];
  }
  float qsum[GPL];
#pragma unroll
  for (int k = 0; k < GPL; ++k) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32 / GPL; ++i) a += qv[(32 / GPL) * k + i];
    qsum[k] = a;
  }
  // twice the table byte offset per step, 8 * (8 sub + ((b + tt) mod 8)): a
  // byte permute puts the token's byte above it (256 v + 8 p) and one shift
  // gives the LDS address 128 v + 4 p of entry p of row v
  uint32_t rq[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) rq[b] = 8u * (uint32_t)(8 * sub + ((b + tt) & 7));
  const uint32_t swap_mask = 0u - (uint32_t)((tt >> 2) & 1);
  const uint32_t rot_sh = 8u * (uint32_t)(tt & 3);
  __syncthreads();

  auto score = [&](const RsTok<GPL>& tk) -> float {
    // INT4 part: nibble e of word k is channel 8 k + e; the low nibbles
    // (even e) and high nibbles (odd e) are taken a byte at a time
    float acc[GPL];
#pragma unroll
    for (int k = 0; k < GPL; ++k) acc[k] = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = tk.c[k] & 0x0F0F0F0Fu;
      const uint32_t hi = (tk.c[k] >> 4) & 0x0F0F0F0Fu;
      const int a = (GPL == 2) ? (k >> 1) : 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        acc[a] = __builtin_fmaf(qv[8 * k + 2 * bb], (float)((lo >> (8 * bb)) & 0xFFu), acc[a]);
        acc[a] = __builtin_fmaf(qv[8 * k + 2 * bb + 1], (float)((hi >> (8 * bb)) & 0xFFu), acc[a]);
      }
    }
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < GPL; ++k) part += tk.s[k] * acc[k] + tk.z[k] * qsum[k];
    // QJL part: the 8 sign bytes rotated by tt mod 8 (words swapped for
    // tt mod 8 >= 4, then a byte shift), one table read per byte
    const uint32_t a0 = tk.w[0] ^ ((tk.w[0] ^ tk.w[1]) & swap_mask);
    const uint32_t a1 = tk.w[1] ^ ((tk.w[0] ^ tk.w[1]) & swap_mask);
    uint32_t x[2];
    x[0] = __builtin_amdgcn_alignbit(a1, a0, rot_sh);
    x[1] = __builtin_amdgcn_alignbit(a0, a1, rot_sh);
    float v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint32_t off =
          __builtin_amdgcn_perm(rq[b], x[b >> 2], 0x07060004u | ((uint32_t)(b & 3) << 8)) >> 1;
      v[b] = *(lds_cfloat_ptr)(uintptr_t)off;
    }
    const float l = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    const float nrm = (float)__builtin_bit_cast(_Float16, (uint16_t)tk.n);
    return part + (kSqrtHalfPi / (float)M) * nrm * l;
  };

  auto finish = [&](const RsTok<GPL> (&tk)[kRsU], int it) {
#pragma unroll
    for (int u = 0; u < kRsU; ++u) {
      const float tot = seg_sum_f32<4>(score(tk[u]));
      const int64_t t = tb + 64 * (it * kRsU + u);
      if (sub == 0 && t < T) scores[gq * T + t] = tot;
    }
  };

#pragma unroll
  for (int it = 0; it < kRsIters; it += 2) {
    RsTok<GPL> kb[kRsU];
    load(kb, std::min(it + 1, kRsIters - 1));
    finish(ka, it);
    if (it + 2 < kRsIters) load(ka, it + 2);
    finish(kb, it + 1);
  }
}

// Scores, any shape: one workgroup per (group, query, 256 tokens), one token
// per thread; q . k_hat from the reconstructed values (binary32 fused
// multiply-adds) and the estimator over the m sign bits with y in LDS.
constexpr int kRsGenTok = 256;

template <typename TQ, typename TS>
__global__ __launch_bounds__(256) void scores_residual_generic_kernel(
    const TQ* __restrict__ q, int nq, const TS* __restrict__ S, int m, int d, int g,
    const uint8_t* __restrict__ codes, const float* __restrict__ steps,
    const float* __restrict__ offsets, const uint32_t* __restrict__ bits,
    const uint16_t* __restrict__ norms, int64_t T, int64_t tiles, float* __restrict__ scores) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  float* y = reinterpret_cast<float*>(lds_raw);     // m
  float* qf = y + kMaxM;                             // d
  float* qs = qf + kMaxDecodeD;                      // staging
  const int64_t gq = blockIdx.x / tiles;
  const int64_t tile = blockIdx.x % tiles;
  const int64_t grp = gq / nq;
  const TQ* qg = q + gq * d;
  project_query_block<TS, TQ>(S, qg, m, d, qs, y);
  for (int i = threadIdx.x; i < d; i += blockDim.x) qf[i] = to_f32(qg[i]);
  __syncthreads();
  const int64_t t = tile * kRsGenTok + threadIdx.x;
  if (t >= T) return;
  const int64_t row = grp * T + t;
  const uint8_t* cr = codes + row * (d / 2);
  const float* sr = steps + row * (d / g);
  const float* zr = offsets + row * (d / g);
  float a = 0.0f;
  for (int j = 0; j < d; ++j) {
    const uint32_t c = (cr[j >> 1] >> (4 * (j & 1))) & 0xFu;
    a = __builtin_fmaf(qf[j], recon4((float)c, sr[j / g], zr[j / g]), a);
  }
  const uint32_t* wr = bits + row * (m / 32);
  float l = 0.0f;
  for (int i = 0; i < m; ++i) l += ((wr[i >> 5] >> (i & 31)) & 1u) ? y[i] : -y[i];
  const float nrm = (float)__builtin_bit_cast(_Float16, norms[row]);
  scores[gq * T + t] = a + (kSqrtHalfPi / (float)m) * nrm * l;
}

template <typename TQ>
static hipError_t scores_residual_fast(const TQ* q, int64_t groups, int nq, const _Float16* S,
                                       int g, const uint8_t* codes, const float* steps,
                                       const float* offsets, const uint32_t* bits,
                                       const uint16_t* norms, int64_t T, float* scores,
                                       hipStream_t st) {
  const size_t lds = (size_t)(kRsLutFloats + 512) * sizeof(float);
  const int64_t tiles = (T + kRsTile - 1) / kRsTile;
  const int64_t per_group = tiles * nq;
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / per_group);
  constexpr int D = 128, M = 256;
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ngr = std::min(max_groups, groups - g0);
    const unsigned blocks = (unsigned)(ngr * per_group);
    const TQ* qp = q + g0 * nq * D;
    const uint8_t* cp = codes + g0 * T * (D / 2);
    const float* sp = steps + g0 * T * (D / g);
    const float* zp = offsets + g0 * T * (D / g);
    const uint32_t* bp = bits + g0 * T * (M / 32);
    const uint16_t* np = norms + g0 * T;
    float* op = scores + g0 * nq * T;
    switch (g) {
      case 16: hipLaunchKernelGGL((scores_residual_kernel<TQ, 16>), dim3(blocks), dim3(kRsThreads), lds, st, qp, nq, S, cp, sp, zp, bp, np, T, tiles, op); break;
      case 32: hipLaunchKernelGGL((scores_residual_kernel<TQ, 32>), dim3(blocks), dim3(kRsThreads), lds, st, qp, nq, S, cp, sp, zp, bp, np, T, tiles, op); break;
      case 64: hipLaunchKernelGGL((scores_residual_kernel<TQ, 64>), dim3(blocks), dim3(kRsThreads), lds, st, qp, nq, S, cp, sp, zp, bp, np, T, tiles, op); break;
      default: hipLaunchKernelGGL((scores_residual_kernel<TQ, 128>), dim3(blocks), dim3(kRsThreads), lds, st, qp, nq, S, cp, sp, zp, bp, np, T, tiles, op); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TQ, typename TS>
static hipError_t scores_residual_generic(const TQ* q, int64_t groups, int nq, const TS* S, int m,
                                          int d, int g, const uint8_t* codes, const float* steps,
                                          const float* offsets, const uint32_t* bits,
                                          const uint16_t* norms, int64_t T, float* scores,
                                          hipStream_t st) {
  const size_t lds = (size_t)(kMaxM + kMaxDecodeD + kProjQChunk) * sizeof(float);
  const int64_t tiles = (T + kRsGenTok - 1) / kRsGenTok;
  const int64_t per_group = tiles * nq;
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / per_group);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ngr = std::min(max_groups, groups - g0);
    const unsigned blocks = (unsigned)(ngr * per_group);
    hipLaunchKernelGGL((scores_residual_generic_kernel<TQ, TS>), dim3(blocks), dim3(256), lds, st,
                       q + g0 * nq * d, nq, S, m, d, g, codes + g0 * T * (d / 2),
                       steps + g0 * T * (d / g), offsets + g0 * T * (d / g),
                       bits + g0 * T * (m / 32), norms + g0 * T, T, tiles, scores + g0 * nq * T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_scores_residual(const void* q, int q_f16, int64_t groups, int nq, const void* S,
                                  int S_f16, int m, int g, const uint8_t* codes,
                                  const float* steps, const float* offsets, const uint32_t* bits,
                                  const uint16_t* norms, int64_t T, int d, float* scores,
                                  hipStream_t st) {
  if (S_f16 && d == 128 && m == 256 && (g == 16 || g == 32 || g == 64 || g == 128)) {
    const _Float16* Sh = static_cast<const _Float16*>(S);
    if (q_f16)
      return scores_residual_fast(static_cast<const _Float16*>(q), groups, nq, Sh, g, codes, steps,
                                  offsets, bits, norms, T, scores, st);
    return scores_residual_fast(static_cast<const float*>(q), groups, nq, Sh, g, codes, steps,
                                offsets, bits, norms, T, scores, st);
  }
  if (q_f16) {
    const _Float16* qh = static_cast<const _Float16*>(q);
    if (S_f16)
      return scores_residual_generic(qh, groups, nq, static_cast<const _Float16*>(S), m, d, g,
                                     codes, steps, offsets, bits, norms, T, scores, st);
    return scores_residual_generic(qh, groups, nq, static_cast<const float*>(S), m, d, g, codes,
                                   steps, offsets, bits, norms, T, scores, st);
  }
  const float* qf = static_cast<const float*>(q);
  if (S_f16)
    return scores_residual_generic(qf, groups, nq, static_cast<const _Float16*>(S), m, d, g, codes,
                                   steps, offsets, bits, norms, T, scores, st);
  return scores_residual_generic(qf, groups, nq, static_cast<const float*>(S), m, d, g, codes,
                                 steps, offsets, bits, norms, T, scores, st);
}

}  // namespace kvq
