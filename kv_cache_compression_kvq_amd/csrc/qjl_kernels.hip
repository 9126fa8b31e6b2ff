// QJL key sketch and asymmetric score for gfx950.
//
// Method: "QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with
// Zero Overhead" (arXiv 2406.03482), abstract: keys are compressed to the
// signs of a Gaussian JL projection (no stored quantization constants) and a
// query's inner product with a key is estimated from the query's unquantized
// projection and the key's sign bits, which is unbiased.  With S [m, d],
// y = S q and bits b of S k, the estimate is
//   sqrt(pi/2) / m * ||k|| * sum_i (2 b_i - 1) y_i.
//
// Sketch (fp16 keys): P = K S^T is a dense contraction with K streamed from
// HBM once and S (<= 64 KiB) resident in LDS, so it runs on fp16 matrix
// cores: v_mfma_f32_32x32x16_f16 with S as the A operand (32 projections x
// 16 channels) and K^T as the B operand (16 channels x 32 tokens).  Products
// of binary16 values are exact in binary32 and the accumulation is binary32.
// S rows are permuted inside each 32-row tile so that lane (token j, half h)
// finds projections 16h .. 16h+15 of that tile in its accumulator registers
// 0..15; its sign word is then built with shift-and-insert steps and one
// exchange with the other half.
//
// Score: per query, y = S q goes to LDS and is expanded into one 256-entry
// table per byte of the sign words:
//   T_p[v] = sum_{j<8} (bit j of v ? +1 : -1) * y_{8p+j},
// so a token costs one table lookup per 8 bits (for m = 256 in a layout
// whose lookups never share an LDS bank within a half-wave).  For m = 256 a
// workgroup takes one tile of a group's tokens and scores all of the group's
// queries against it; other shapes take one (group, query, tile).
#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_qjl_device.h"
#include "kvq_qjl_stream.h"

#include <algorithm>
#include <cmath>

namespace kvq {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Sketch, fp16 keys on MFMA.  KS = d / 16 K-steps; MT = m / 32 projection
// tiles, a multiple of 8 (MT == 0: runtime m, words stored as they are
// produced).  Each wave owns NT x 32 tokens per iteration and loops over
// token tiles.  d = 128 with m = 256: one 32-token tile per wave iteration,
// two in flight, in 768-thread workgroups at three waves per SIMD (144
// registers): more waves hide more of the key stream's latency than a second
// tile per wave does (about 5 % faster, the same words).  Other shapes:
// token tiles of 32 per wave iteration, two, or one when d = 256 would
// otherwise spill, in 512-thread workgroups at two waves per SIMD.
template <int KS, int MT> constexpr bool sketch_wide() { return KS == 8 && MT == 8; }
template <int KS, int MT> constexpr int sketch_nt() {
  return sketch_wide<KS, MT>() ? 1 : (KS <= 8 ? 2 : 1);
}
// Key tiles in flight per wave (a ring of register buffers): two at d = 128,
// m = 256; else four single tiles up to d = 192, two above (four would spill
// registers).
template <int KS, int MT> constexpr int sketch_ring() {
  return sketch_wide<KS, MT>() ? 2 : (sketch_nt<KS, MT>() == 1 && KS <= 12 ? 4 : 2);
}
template <int KS, int MT> constexpr int sketch_threads() { return sketch_wide<KS, MT>() ? 768 : 512; }
template <int KS, int MT> constexpr int sketch_waves_per_eu() { return sketch_wide<KS, MT>() ? 3 : 2; }

// Sign words of projection tile mt (32 projections) for the NT x 32 tokens
// of a wave: P = S_tile K^T on fp16 MFMA, then bit = [P >= 0].  Accumulator
// r of lane (token j, half h) holds projection 32 mt + 16 h + r (the rows of
// S are permuted in LDS); each step shifts the sign bit of one accumulator in
// (v_alignbit), MSB first, and the bits are inverted at the end.  A zero
// projection is +0 here (the accumulation starts from +0), so it gives bit 1.
// Both halves of the wave return the token's full 32-bit word (the halves'
// 16-bit parts are exchanged with v_permlane32_swap).

// Multiplies of projection tile mt for the NT x 32 tokens of a wave:
// P = S_tile K^T on fp16 MFMA into acc.
template <int KS, int NT>
__device__ __forceinline__ void sketch_tile_mfma(const f16x8* sfrag, int mt, int lane,
                                                 const f16x8 (&b)[NT][KS], f32x16 (&acc)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const f16x8 a = sfrag[(mt * KS + ks) * 64 + lane];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b[nt][ks], acc[nt], 0, 0, 0);
  }
}

// Sign word of each token from the accumulators of one projection tile.
template <int NT>
__device__ __forceinline__ void sketch_tile_signs(const f32x16 (&acc)[NT], uint32_t (&full)[NT]) {
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    uint32_t sb = 0;
#pragma unroll
    for (int r = 15; r >= 0; --r) {
      const float pr = acc[nt][r];   // copy first: bit-casting the vector element in place reads element 0
      sb = __builtin_amdgcn_alignbit(sb, __builtin_bit_cast(uint32_t, pr), 31);
    }
    uint32_t lo, hi;
    halves_u32(~sb & 0xFFFFu, lo, hi);
    full[nt] = lo | (hi << 16);
  }
}

template <int KS, int NT>
__device__ __forceinline__ void sketch_tile_words(const f16x8* sfrag, int mt, int lane,
                                                  const f16x8 (&b)[NT][KS], uint32_t (&full)[NT]) {
  f32x16 acc[NT];
  sketch_tile_mfma<KS, NT>(sfrag, mt, lane, b, acc);
  sketch_tile_signs<NT>(acc, full);
}

constexpr int kSketchThreads = 512;
constexpr int kSketchWaves = kSketchThreads / 64;

// A launch computes projection tiles [mt0, mt0 + m_rt / 32) of every row
// (sign words mt0 .. of words_total per row); S larger than a workgroup's
// LDS takes several launches, and the one with mt0 == 0 writes the norms.
template <int KS, int MT>
__global__ __launch_bounds__((sketch_threads<KS, MT>()))
__attribute__((amdgpu_waves_per_eu((sketch_waves_per_eu<KS, MT>()))))
void sketch_mfma_kernel(const _Float16* __restrict__ k,
                                                          int64_t rows,
                                                          const _Float16* __restrict__ S,
                                                          int m_rt, uint32_t* __restrict__ bits,
                                                          uint16_t* __restrict__ norms,
                                                          int mt0, int words_total) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  constexpr int TH = sketch_threads<KS, MT>();
  constexpr int kWaves = TH / 64;
  f16x8* sfrag = reinterpret_cast<f16x8*>(lds_raw);
  constexpr int D = KS * 16;
  const int mt_count = MT > 0 ? MT : m_rt / 32;
  const int words = MT > 0 ? MT : words_total;  // sign words per token
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  // S -> LDS in fragment order: fragment (mt, ks), lane l holds
  // S[32 mt + perm(l % 32)][16 ks + 8 (l / 32) .. + 8].
  const int nfrag_lanes = mt_count * KS * 64;
  for (int idx = tid; idx < nfrag_lanes; idx += TH) {
    const int l = idx & 63;
    const int frag = idx >> 6;
    const int mt = frag / KS, ks = frag % KS;
    const int srow = 32 * (mt0 + mt) + sketch_row_perm(l & 31);
    sfrag[idx] = *reinterpret_cast<const f16x8*>(S + (int64_t)srow * D + 16 * ks + 8 * (l >> 5));
  }
  // tiles handed out so far (after the S fragments)
  int* next_tile = reinterpret_cast<int*>(sfrag + nfrag_lanes);
  constexpr int RING = sketch_ring<KS, MT>();
  if (tid == 0) *next_tile = RING * kWaves;
  __syncthreads();

  constexpr int kSketchNT = sketch_nt<KS, MT>();
  const int64_t tiles = (rows + 32 * kSketchNT - 1) / (32 * kSketchNT);

  // B fragments of one token tile: lane (token j, half h) holds channels
  // 16 ks + 8 h .. + 8 of token 32 nt + j.  The loads are unconditional
  // (tokens past the end re-read the last row and are not stored): a load
  // under a branch would make the compiler's wait counts conservative and
  // serialise the prefetch with the multiplies.
  auto load = [&](f16x8 (&b)[kSketchNT][KS], int64_t tile) {
    const int64_t tok0 = tile * (32 * kSketchNT);
#pragma unroll
    for (int nt = 0; nt < kSketchNT; ++nt) {
      const int64_t tok = std::min<int64_t>(tok0 + 32 * nt + col, rows - 1);
      const _Float16* kr = k + tok * D + 8 * h;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) b[nt][ks] = *reinterpret_cast<const f16x8*>(kr + 16 * ks);
    }
  };

  auto process = [&](const f16x8 (&b)[kSketchNT][KS], int64_t tile) {
    const int64_t tok0 = tile * (32 * kSketchNT);
    // S fragments are re-read from LDS for every tile (an opaque offset
    // stops the compiler from hoisting all of them into registers)
    int off = 0;
    asm volatile("" : "+v"(off));
    const f16x8* sf = sfrag + off;
    // norms: this lane holds half of its token's channels; packed fp16
    // products (exact in binary32) summed in binary32
    float ss[kSketchNT];
#pragma unroll
    for (int nt = 0; nt < kSketchNT; ++nt) {
      float acc = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 v2 = {b[nt][ks][2 * e], b[nt][ks][2 * e + 1]};
          acc = __builtin_amdgcn_fdot2(v2, v2, acc, false);
        }
      ss[nt] = acc;
    }
#pragma unroll
    for (int nt = 0; nt < kSketchNT; ++nt) {
      uint32_t slo, shi;
      halves_u32(__builtin_bit_cast(uint32_t, ss[nt]), slo, shi);
      const float tot = __builtin_bit_cast(float, slo) + __builtin_bit_cast(float, shi);
      const int64_t tok = tok0 + 32 * nt + col;
      if (h == 0 && tok < rows && mt0 == 0) norms[tok] = f32_to_f16_bits(__builtin_sqrtf(tot));
    }
    if constexpr (MT > 0) {
      // unrolled so the words stay in registers; the scheduling barrier
      // keeps each tile's S-fragment reads inside its own iteration
      uint32_t wbuf[kSketchNT][MT];
      // two accumulator sets: the sign words of tile mt - 1 are taken while
      // the multiplies of tile mt run, interleaved per k-step (an S fragment
      // read two k-steps ahead, the step's multiplies, five sign-extraction
      // instructions), so the matrix cores do not wait for the extraction
      f32x16 acc0[kSketchNT], acc1[kSketchNT];
      __builtin_amdgcn_sched_barrier(0);
      sketch_tile_mfma<KS, kSketchNT>(sf, 0, lane, b, acc0);
#pragma unroll
      for (int mt = 1; mt <= MT; ++mt) {
        __builtin_amdgcn_sched_barrier(0);
        uint32_t f[kSketchNT];
        if (mt & 1) {
          if (mt < MT) sketch_tile_mfma<KS, kSketchNT>(sf, mt, lane, b, acc1);
          sketch_tile_signs<kSketchNT>(acc0, f);
        } else {
          if (mt < MT) sketch_tile_mfma<KS, kSketchNT>(sf, mt, lane, b, acc0);
          sketch_tile_signs<kSketchNT>(acc1, f);
        }
        if (mt < MT) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);        // LDS reads
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, kSketchNT, 0);   // MFMA
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);      // VALU
          }
        }
#pragma unroll
        for (int nt = 0; nt < kSketchNT; ++nt) wbuf[nt][mt - 1] = f[nt];
      }
      // half h stores words [h * MT/2, (h + 1) * MT/2) of its token
      constexpr int HALF = MT / 2;
#pragma unroll
      for (int nt = 0; nt < kSketchNT; ++nt) {
        const int64_t tok = tok0 + 32 * nt + col;
        if (tok < rows) {
          uint32_t* dst = bits + tok * MT + h * HALF;
          // lane-mask blend rather than a select, which the compiler would
          // turn into a dynamically indexed (scratch) load of wbuf
          const uint32_t lo_mask = h == 0 ? 0xFFFFFFFFu : 0u;
#pragma unroll
          for (int v4 = 0; v4 < HALF / 4; ++v4) {
            u32x4 val;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              val[j] = (wbuf[nt][4 * v4 + j] & lo_mask) | (wbuf[nt][HALF + 4 * v4 + j] & ~lo_mask);
            *reinterpret_cast<u32x4*>(dst + 4 * v4) = val;
          }
        }
      }
    } else {
#pragma unroll 1
      for (int mt = 0; mt < mt_count; ++mt) {
        uint32_t f[kSketchNT];
        sketch_tile_words<KS, kSketchNT>(sf, mt, lane, b, f);
#pragma unroll
        for (int nt = 0; nt < kSketchNT; ++nt) {
          const int64_t tok = tok0 + 32 * nt + col;
          if (h == 0 && tok < rows) bits[tok * words + mt0 + mt] = f[nt];
        }
      }
    }
  };

  // A workgroup takes a contiguous range of the tiles; its waves take tiles
  // w, w + W, ... (W waves, RING of them each) first, then claim the next
  // free tile of the range from an LDS counter as they refill a buffer, so
  // waves that the scheduler serves faster take more tiles (with a fixed
  // stride per wave the last tiles of a workgroup ran on a few waves).  RING
  // token tiles in flight per wave: a ring of register buffers, each
  // refilled (unconditionally, clamped past the range) right after its
  // tile's multiplies are issued; claims only grow, so a wave stops at its
  // first tile past the range.
  const int64_t per_wg = (tiles + gridDim.x - 1) / gridDim.x;
  const int64_t wg_first = (int64_t)blockIdx.x * per_wg;
  const int64_t wg_count = std::min<int64_t>(per_wg, tiles - wg_first);
  if (wg_count <= 0) return;
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(next_tile, 1);
    return (int64_t)__builtin_amdgcn_readfirstlane(v);
  };
  f16x8 bq[RING][kSketchNT][KS];
  int64_t idx[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r) {
    idx[r] = wave + r * kWaves;
    load(bq[r], wg_first + std::min(idx[r], wg_count - 1));
  }
  // the slots in order, each refilled right after its tile is processed
  // (written out: the buffers are indexed by constants only)
  static_assert(RING == 2 || RING == 4, "ring of 2 or 4 tiles");
  if (idx[0] >= wg_count) return;
  for (;;) {
    process(bq[0], wg_first + idx[0]);
    idx[0] = claim();
    load(bq[0], wg_first + std::min(idx[0], wg_count - 1));
    if (idx[1] >= wg_count) return;
    process(bq[1], wg_first + idx[1]);
    idx[1] = claim();
    load(bq[1], wg_first + std::min(idx[1], wg_count - 1));
    if constexpr (RING == 4) {
      if (idx[2] >= wg_count) return;
      process(bq[2], wg_first + idx[2]);
      idx[2] = claim();
      load(bq[2], wg_first + std::min(idx[2], wg_count - 1));
      if (idx[3] >= wg_count) return;
      process(bq[3], wg_first + idx[3]);
      idx[3] = claim();
      load(bq[3], wg_first + std::min(idx[3], wg_count - 1));
    }
    if (idx[0] >= wg_count) return;
  }
}

// ---------------------------------------------------------------------------
// Sketch, fp32 keys and S, on fp16 matrix cores.  Each row of S and each key
// is scaled by a power of two (exact; it does not change a projection's
// sign) so that its largest magnitude lies in [2^14, 2^15), then split into
// two binary16 parts: hi = the value with its 13 low significand bits
// cleared, lo = the exact remainder rounded toward zero, so hi + lo is within
// 2^-20 relative (2^-24 absolute below the binary16 normal range) of the
// scaled value.  P = S_hi k_hi + S_hi k_lo + S_lo k_hi (three MFMAs per
// K-step, fp32 accumulation) then differs from the exact projection by a few
// 2^-20 sum_j |S_ij k_j| <= 2^-18 ||S_i|| ||k||, well inside the 1e-4 sign
// band.  The norm is accumulated from the binary32 key values.  One 32-token
// tile per wave iteration; S's hi and lo fragments (projection tiles
// [mt0, mt0 + mt_pass)) are resident in LDS.
template <int KS>
constexpr int split_ring() { return KS <= 8 ? 2 : 1; }

// hi / lo binary16 parts of two scaled binary32 values.
__device__ __forceinline__ void split2(float v0, float v1, _Float16& h0, _Float16& h1,
                                       _Float16& l0, _Float16& l1) {
  const float a0 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v0) & 0xFFFFE000u);
  const float a1 = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v1) & 0xFFFFE000u);
  const auto ph = __builtin_amdgcn_cvt_pkrtz(a0, a1);
  const auto pl = __builtin_amdgcn_cvt_pkrtz(v0 - a0, v1 - a1);
  h0 = ph[0];
  h1 = ph[1];
  l0 = pl[0];
  l1 = pl[1];
}

// The same lane value of the other half of the wave (lane l <-> l ^ 32).
__device__ __forceinline__ float other_half(float v, int h) {
  uint32_t lo, hi;
  halves_u32(__builtin_bit_cast(uint32_t, v), lo, hi);
  return __builtin_bit_cast(float, h == 0 ? hi : lo);
}

template <int KS>
__global__ __launch_bounds__(kSketchThreads) __attribute__((amdgpu_waves_per_eu(2)))
void sketch_split_kernel(const float* __restrict__ k, int64_t rows, const float* __restrict__ S,
                         int mt_pass, uint32_t* __restrict__ bits, uint16_t* __restrict__ norms,
                         int mt0, int words_total) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  constexpr int D = KS * 16;
  const int nfrag_lanes = mt_pass * KS * 64;
  f16x8* shi = reinterpret_cast<f16x8*>(lds_raw);
  f16x8* slo = shi + nfrag_lanes;
  int* rsc = reinterpret_cast<int*>(slo + nfrag_lanes);     // [32 mt_pass] row exponents
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  // scale exponent of every S row of this pass
  for (int r = tid; r < 32 * mt_pass; r += kSketchThreads) {
    const float* sr = S + (int64_t)(32 * mt0 + r) * D;
    float a = 0.0f;
    for (int j = 0; j < D; j += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sr + j);
      a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                                             __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3]))));
    }
    rsc[r] = 15 - __builtin_amdgcn_frexp_expf(a);
  }
  __syncthreads();
  // S -> LDS in fragment order (as the fp16 sketch), hi and lo parts
  for (int idx = tid; idx < nfrag_lanes; idx += kSketchThreads) {
    const int l = idx & 63;
    const int frag = idx >> 6;
    const int mt = frag / KS, ks = frag % KS;
    const int rloc = 32 * mt + sketch_row_perm(l & 31);
    const float* sp = S + (int64_t)(32 * mt0 + rloc) * D + 16 * ks + 8 * (l >> 5);
    const f32x4 u = *reinterpret_cast<const f32x4*>(sp);
    const f32x4 w = *reinterpret_cast<const f32x4*>(sp + 4);
    const int e = rsc[rloc];
    const float v[8] = {u[0], u[1], u[2], u[3], w[0], w[1], w[2], w[3]};
    f16x8 hv, lv;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      _Float16 h0, h1, l0, l1;
      split2(__builtin_amdgcn_ldexpf(v[i], e), __builtin_amdgcn_ldexpf(v[i + 1], e), h0, h1, l0, l1);
      hv[i] = h0;
      hv[i + 1] = h1;
      lv[i] = l0;
      lv[i + 1] = l1;
    }
    shi[idx] = hv;
    slo[idx] = lv;
  }
  __syncthreads();

  const int64_t tiles = (rows + 31) / 32;
  // lane (token j, half h) holds channels 16 ks + 8 h .. + 8 of token j;
  // loads unconditional (clamped to the last row past the end)
  auto load = [&](f32x4 (&b)[KS][2], int64_t tile) {
    const int64_t tok = std::min<int64_t>(tile * 32 + col, rows - 1);
    const float* kr = k + tok * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      b[ks][0] = *reinterpret_cast<const f32x4*>(kr + 16 * ks);
      b[ks][1] = *reinterpret_cast<const f32x4*>(kr + 16 * ks + 4);
    }
  };

  auto process = [&](const f32x4 (&b)[KS][2], int64_t tile) {
    const int64_t tok = tile * 32 + col;
    int off = 0;
    asm volatile("" : "+v"(off));
    const f16x8* sh = shi + off;
    const f16x8* sl = slo + off;
    float ss = 0.0f, am = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ss = __builtin_fmaf(b[ks][p][e], b[ks][p][e], ss);
          am = __builtin_fmaxf(am, __builtin_fabsf(b[ks][p][e]));
        }
    ss += other_half(ss, h);
    am = __builtin_fmaxf(am, other_half(am, h));
    if (h == 0 && tok < rows && mt0 == 0) norms[tok] = f32_to_f16_bits(__builtin_sqrtf(ss));
    const int sc = 15 - __builtin_amdgcn_frexp_expf(am);
    f16x8 bh[KS], bl[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        _Float16 h0, h1, l0, l1;
        split2(__builtin_amdgcn_ldexpf(b[ks][i >> 2][i & 3], sc),
               __builtin_amdgcn_ldexpf(b[ks][(i + 1) >> 2][(i + 1) & 3], sc), h0, h1, l0, l1);
        bh[ks][i] = h0;
        bh[ks][i + 1] = h1;
        bl[ks][i] = l0;
        bl[ks][i + 1] = l1;
      }
#pragma unroll 1
    for (int mt = 0; mt < mt_pass; ++mt) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8 ah = sh[(mt * KS + ks) * 64 + lane];
        const f16x8 al = sl[(mt * KS + ks) * 64 + lane];
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl[ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh[ks], acc, 0, 0, 0);
      }
      const f32x16 a1[1] = {acc};
      uint32_t f[1];
      sketch_tile_signs<1>(a1, f);
      if (h == 0 && tok < rows) bits[tok * words_total + mt0 + mt] = f[0];
    }
  };

  constexpr int RING = split_ring<KS>();
  const int64_t stride = (int64_t)gridDim.x * kSketchWaves;
  const int64_t first = (int64_t)blockIdx.x * kSketchWaves + wave;
  if (first >= tiles) return;
  f32x4 bq[RING][KS][2];
#pragma unroll
  for (int r = 0; r < RING; ++r) load(bq[r], std::min(first + r * stride, tiles - 1));
  for (int64_t t0 = first;; t0 += RING * stride) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const int64_t t = t0 + r * stride;
      process(bq[r], t);
      if (t + stride >= tiles) return;
      load(bq[r], std::min(t + RING * stride, tiles - 1));
    }
  }
}

// ---------------------------------------------------------------------------
// Sketch, d > 256 (beyond the MFMA kernels' register-resident K-steps): one
// thread per (row, sign word), 32 binary32 dot products each; the word-0
// thread also writes the norm.
template <typename T>
__global__ __launch_bounds__(256) void sketch_generic_kernel(const T* __restrict__ k, int64_t rows,
                                                             int d, const T* __restrict__ S, int m,
                                                             uint32_t* __restrict__ bits,
                                                             uint16_t* __restrict__ norms) {
  const int words = m / 32;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / words;
  const int w = (int)(gid % words);
  if (row >= rows) return;
  const T* kr = k + row * d;
  uint32_t word = 0;
  for (int i = 0; i < 32; ++i) {
    const T* sr = S + (int64_t)(32 * w + i) * d;
    float p = 0.0f;
    for (int j = 0; j < d; ++j) p = __builtin_fmaf(to_f32(sr[j]), to_f32(kr[j]), p);
    word |= (p >= 0.0f ? 1u : 0u) << i;
  }
  bits[row * words + w] = word;
  if (w == 0) {
    float acc = 0.0f;
    for (int j = 0; j < d; ++j) {
      const float v = to_f32(kr[j]);
      acc = __builtin_fmaf(v, v, acc);
    }
    norms[row] = f32_to_f16_bits(__builtin_sqrtf(acc));
  }
}

// Persistent grid: exactly the workgroups that fit on the device at once
// (registers and LDS both limit it), each striding over the token tiles.
template <typename Kernel>
static hipError_t persistent_blocks(Kernel kernel, size_t lds, int64_t tiles,
                                    const DeviceInfo& dev, int64_t* blocks,
                                    int threads = kSketchThreads) {
  hipError_t e = allow_dynamic_lds(kernel, lds);
  if (e != hipSuccess) return e;
  int per_cu = 0;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
  if (e != hipSuccess) return e;
  const int waves = threads / 64;
  const int64_t want = (tiles + waves - 1) / waves;
  const int64_t cap = (int64_t)dev.cus * std::max(1, per_cu);
  *blocks = std::max<int64_t>(1, std::min(want, cap));
  return hipSuccess;
}

// Projection tiles per launch when S's fragments (bytes_per_tile each) must
// fit in `lds` bytes: the m / 32 tiles in as few, equal launches as fit.
static int tiles_per_pass(int mt_total, size_t bytes_per_tile, size_t lds) {
  const int fit = std::max<int>(1, (int)(lds / bytes_per_tile));
  const int passes = (mt_total + fit - 1) / fit;
  return (mt_total + passes - 1) / passes;
}

template <int KS, int MT>
static hipError_t sketch_mfma_launch(const _Float16* k, int64_t rows, const _Float16* S, int m,
                                     uint32_t* bits, uint16_t* norms, const DeviceInfo& dev,
                                     hipStream_t st) {
  constexpr int kSketchNT = sketch_nt<KS, MT>();
  constexpr int TH = sketch_threads<KS, MT>();
  const int64_t tiles = (rows + 32 * kSketchNT - 1) / (32 * kSketchNT);
  const int mt_total = m / 32;
  const size_t tile_bytes = (size_t)32 * KS * 16 * sizeof(_Float16);
  const int per = MT > 0 ? MT : tiles_per_pass(mt_total, tile_bytes, dev.lds_per_block - 16);
  for (int mt0 = 0; mt0 < mt_total; mt0 += per) {
    const int mtp = std::min(per, mt_total - mt0);
    const size_t lds = (size_t)mtp * tile_bytes + 16;   // S fragments + the tile counter
    int64_t blocks = 0;
    hipError_t e = persistent_blocks(sketch_mfma_kernel<KS, MT>, lds, tiles, dev, &blocks, TH);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sketch_mfma_kernel<KS, MT>), dim3((unsigned)blocks), dim3(TH),
                       lds, st, k, rows, S, 32 * mtp, bits, norms, mt0, mt_total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KS>
static hipError_t sketch_split_launch(const float* k, int64_t rows, const float* S, int m,
                                      uint32_t* bits, uint16_t* norms, const DeviceInfo& dev,
                                      hipStream_t st) {
  const int64_t tiles = (rows + 31) / 32;
  const int mt_total = m / 32;
  // hi and lo fragments plus one exponent per S row, per projection tile
  const size_t tile_bytes = (size_t)2 * 32 * KS * 16 * sizeof(_Float16) + 32 * sizeof(int);
  const int per = tiles_per_pass(mt_total, tile_bytes, dev.lds_per_block);
  for (int mt0 = 0; mt0 < mt_total; mt0 += per) {
    const int mtp = std::min(per, mt_total - mt0);
    const size_t lds = (size_t)mtp * tile_bytes;
    int64_t blocks = 0;
    hipError_t e = persistent_blocks(sketch_split_kernel<KS>, lds, tiles, dev, &blocks);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sketch_split_kernel<KS>), dim3((unsigned)blocks), dim3(kSketchThreads), lds,
                       st, k, rows, S, mtp, bits, norms, mt0, mt_total);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int KS>
static hipError_t sketch_by_ks(const void* k, int k_f16, int64_t rows, const void* S, int m,
                               uint32_t* bits, uint16_t* norms, const DeviceInfo& dev,
                               hipStream_t st) {
  if (k_f16)
    return sketch_mfma_launch<KS, 0>(static_cast<const _Float16*>(k), rows,
                                     static_cast<const _Float16*>(S), m, bits, norms, dev, st);
  return sketch_split_launch<KS>(static_cast<const float*>(k), rows, static_cast<const float*>(S),
                                 m, bits, norms, dev, st);
}

// Largest head dimension whose K-steps the MFMA sketches hold in registers.
constexpr int kSketchMfmaMaxD = 256;

hipError_t launch_qjl_sketch(const void* k, int k_f16, int64_t rows, int d, const void* S, int m,
                             uint32_t* bits, uint16_t* norms, const DeviceInfo& dev,
                             hipStream_t st) {
  if (k_f16 && d == 128 && m == 256 && dev.lds_per_block >= (size_t)m * d * sizeof(_Float16) + 16)
    return sketch_mfma_launch<8, 8>(static_cast<const _Float16*>(k), rows,
                                    static_cast<const _Float16*>(S), m, bits, norms, dev, st);
  switch (d) {
    case 16: return sketch_by_ks<1>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 32: return sketch_by_ks<2>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 48: return sketch_by_ks<3>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 64: return sketch_by_ks<4>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 80: return sketch_by_ks<5>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 96: return sketch_by_ks<6>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 112: return sketch_by_ks<7>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 128: return sketch_by_ks<8>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 144: return sketch_by_ks<9>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 160: return sketch_by_ks<10>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 176: return sketch_by_ks<11>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 192: return sketch_by_ks<12>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 208: return sketch_by_ks<13>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 224: return sketch_by_ks<14>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 240: return sketch_by_ks<15>(k, k_f16, rows, S, m, bits, norms, dev, st);
    case 256: return sketch_by_ks<16>(k, k_f16, rows, S, m, bits, norms, dev, st);
    default: break;
  }
  static_assert(kSketchMfmaMaxD == 256, "the switch above covers d = 16 .. 256");
  // d > 256: the generic kernel, launched in row slices to bound the grid
  const int64_t rows_per = std::max<int64_t>(1, (int64_t(1) << 30) / (m / 32));
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per) {
    const int64_t nr = std::min(rows_per, rows - r0);
    const int64_t nb = (nr * (m / 32) + 255) / 256;
    if (k_f16)
      hipLaunchKernelGGL(sketch_generic_kernel<_Float16>, dim3((unsigned)nb), dim3(256), 0, st,
                         static_cast<const _Float16*>(k) + r0 * d, nr, d,
                         static_cast<const _Float16*>(S), m, bits + r0 * (m / 32), norms + r0);
    else
      hipLaunchKernelGGL(sketch_generic_kernel<float>, dim3((unsigned)nb), dim3(256), 0, st,
                         static_cast<const float*>(k) + r0 * d, nr, d,
                         static_cast<const float*>(S), m, bits + r0 * (m / 32), norms + r0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// QJL scores.  m = 256 (fp16 S, d <= 128): one workgroup per (group, tile of
// TH * kQjlBatch tokens) scores all of the group's queries, each thread
// holding kQjlBatch tokens TH apart in registers.  Other shapes: one
// workgroup per (group, query, tile of kQjlTok tokens), kQjlTokPerThread
// tokens per thread.
constexpr int kQjlBatch = 8;
constexpr int kQjlThreads = 256;
constexpr int kQjlWideThreads = 512;
constexpr int kQjlOneQThreads = 1024;   // one query, caches of more than 4096 tokens
constexpr int kQjlTokPerThread = 16;
constexpr int kQjlTok = kQjlThreads * kQjlTokPerThread;

// LDS: byte tables (rotated layout for m = 256, else [m / 8][256]) | y [m];
// the table area is also the query staging area of the projection, which
// ends before the tables are built.
__host__ __device__ inline size_t qjl_table_lds_floats(int m) {
  const size_t tables = byte_table_floats(m, m == 256);
  return (size_t)m + (tables > (size_t)kProjQChunk ? tables : (size_t)kProjQChunk);
}

// TH: threads per workgroup.  ONEQ: one query per group.  The m = 256
// kernels stay under 128 registers, i.e. four waves per SIMD (two 512-thread
// workgroups with 64 KiB of tables each, or one of 1024 threads, per CU),
// which hides more of the lookups' LDS latency; per-lane token offsets are
// 32-bit from workgroup-uniform bases.
template <typename TS, typename TQ, int W, int TH = kQjlThreads, bool ONEQ = false>
__global__ __launch_bounds__(TH) __attribute__((amdgpu_waves_per_eu(W == 8 ? 4 : 2))) void scores_qjl_kernel(const TQ* __restrict__ q, int nq,
                                                         const TS* __restrict__ S, int m_rt, int d,
                                                         const uint32_t* __restrict__ bits,
                                                         const uint16_t* __restrict__ norms,
                                                         int64_t T, int64_t tiles,
                                                         float* __restrict__ scores) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int m = W > 0 ? 32 * W : m_rt;
  const int words = m / 32;
  // tables first: at LDS address 0 a lookup's address is the byte permute's
  // result plus the instruction offset, with no base to add.  The rotated
  // lookups require it (see rot_lane_base): this kernel declares no static
  // __shared__ data, so its dynamic LDS starts at address 0.
  float* lut = reinterpret_cast<float*>(lds_raw);
  const size_t tfl = byte_table_floats(m, m == 256);
  float* y = lut + (tfl > (size_t)kProjQChunk ? tfl : (size_t)kProjQChunk);
  const float c = kSqrtHalfPi / (float)m;
  if constexpr (W == 8) {
    constexpr int kTile = TH * kQjlBatch;
    // One workgroup per (group, tile): thread i holds tokens i + u TH
    // (u < kQjlBatch), so a wave's step u is 64 consecutive tokens, read as
    // whole lines (issue_rot_words64).  Loads are unconditional (tokens past
    // T re-read the tile's last token and are not stored): loads under a
    // branch make the compiler wait for each one.
    const int64_t g = blockIdx.x / tiles;
    const int64_t tile = blockIdx.x % tiles;
    const int64_t tbase = tile * kTile;
    const int nlive = (int)std::min<int64_t>(kTile, T - tbase);   // tokens of this tile
    const uint32_t* bg = bits + (g * T + tbase) * words;
    const uint16_t* ng = norms + g * T + tbase;
    const int lane = threadIdx.x & 63;
    const int r = lane & 31;
    const int wfirst = (int)threadIdx.x - lane;   // the wave's first token of step 0
    RotWords64 rw[kQjlBatch];
    float nv[kQjlBatch];
    auto load_step = [&](int u) {
      const int tb = wfirst + u * TH;
      issue_rot_words64(bg, tb, nlive - 1, lane, rw[u]);
      const uint32_t nb = 2u * (uint32_t)min(tb + lane, nlive - 1);   // byte offset
      nv[u] = (float)__builtin_bit_cast(
          _Float16, ld_stream(reinterpret_cast<const uint16_t*>(
                        reinterpret_cast<const unsigned char*>(ng) + nb)));
    };
    const TQ* q0 = q + g * nq * d;
    // (this kernel is launched for fp16 S with d <= 128 only)
    if constexpr (ONEQ && sizeof(TS) == 2) {
      // One query: y = S q and the tables first, then the tokens, each wave
      // requesting step u + 1 before it scores step u.  A CU's vector loads
      // return in issue order, so S rows requested behind token loads would
      // wait for HBM: every wave receives its S rows (L2-resident after the
      // first workgroups) before it requests a token, and one step ahead is
      // enough to keep HBM busy (more queues the lookups of later waves
      // behind this wave's loads).
      QueryProjDirect<TQ, 256 / (TH / 64) / 4> pj;
      pj.issue(S, q0, d);
      pj.wait();
      __builtin_amdgcn_sched_barrier(0);
      load_step(0);
      __builtin_amdgcn_sched_barrier(0);
      pj.finish(y, d);
      __syncthreads();
      build_rot_tables(y, lut);
      __syncthreads();
      const uint32_t rq = rot_lane_base(lut, r);
      float* st = scores + g * T + tbase;
#pragma unroll
      for (int u = 0; u < kQjlBatch; ++u) {
        if (u + 1 < kQjlBatch) load_step(u + 1);
        __builtin_amdgcn_sched_barrier(0);
        uint32_t w[8];
        finish_rot_words64(rw[u], w);
        const float acc = rot_lut_sum(w, r, rq);
        const int t = wfirst + u * TH + lane;
        if (t < nlive) st[t] = c * nv[u] * acc;
      }
      return;
    }
    // Several queries of a KV head (grouped-query attention) share one pass
    // over its sign words and norms, which stay in registers: per query, y
    // = S q and the byte tables are rebuilt in LDS, then the tokens are
    // scored.  The tokens are requested once the first query's projection
    // is done (its S rows then do not wait behind them, and its registers
    // are free).
    auto load_tokens = [&]() {
#pragma unroll
      for (int u = 0; u < kQjlBatch; ++u) load_step(u);
    };
    // the words are rotated once (rot_words), back into rw, and serve every
    // query
    auto rotate_all = [&]() {
#pragma unroll
      for (int u = 0; u < kQjlBatch; ++u) {
        uint32_t w[8], x[8];
        finish_rot_words64(rw[u], w);
        rot_words(w, r, x);
        rw[u].x = u32x4{x[0], x[1], x[2], x[3]};
        rw[u].y = u32x4{x[4], x[5], x[6], x[7]};
      }
    };
    auto score_all = [&](float* sg) {
      // opaque per call: the lookup addresses depend only on the words and
      // r, and hoisting all of them out of the query loop would need 256
      // registers
      uint32_t rq = rot_lane_base(lut, r);
      asm volatile("" : "+v"(rq));
      float* st = sg + tbase;
#pragma unroll
      for (int u = 0; u < kQjlBatch; ++u) {
        const int t = wfirst + u * TH + lane;
        const uint32_t x[8] = {rw[u].x[0], rw[u].x[1], rw[u].x[2], rw[u].x[3],
                               rw[u].y[0], rw[u].y[1], rw[u].y[2], rw[u].y[3]};
        const float acc = rot_lut_sum_rotated(x, rq);
        if (t < nlive) st[t] = c * nv[u] * acc;
      }
    };
    if constexpr (sizeof(TS) == 2) {
      project16_lite(S, q0, m, d, lut, y);
      __builtin_amdgcn_sched_barrier(0);
      load_tokens();
      __syncthreads();
      build_rot_tables(y, lut);
      __syncthreads();
      rotate_all();
      score_all(scores + g * nq * T);
      // queries 1 .. nq - 1: the tokens are already in registers
      if constexpr (!ONEQ)
        for (int j = 1; j < nq; ++j) {
          __syncthreads();                     // every lookup of query j - 1 is done
          project16_lite(S, q0 + (int64_t)j * d, m, d, lut, y);
          __syncthreads();
          build_rot_tables(y, lut);
          __syncthreads();
          score_all(scores + (g * nq + j) * T);
        }
    }
    return;
  }
  const int64_t gj = blockIdx.x / tiles;           // (group, query) pair
  const int64_t tile = blockIdx.x % tiles;
  const int64_t g = gj / nq;
  const uint32_t* bg = bits + g * T * words;
  const uint16_t* ng = norms + g * T;
  float* sg = scores + gj * T;
  const int64_t t0 = tile * kQjlTok + threadIdx.x;
  project_query_block(S, q + gj * d, m, d, lut, y);
  __syncthreads();
  build_byte_tables(y, m / 8, lut);
  __syncthreads();
  for (int u = 0; u < kQjlTokPerThread; ++u) {
    const int64_t t = t0 + (int64_t)u * kQjlThreads;
    if (t >= T) break;
    float acc = 0.0f;
    for (int i = 0; i < words; ++i) {
      const uint32_t x = bg[t * words + i];
      acc += lut_sum(lut + i * 1024, &x, 1);
    }
    sg[t] = c * (float)__builtin_bit_cast(_Float16, ng[t]) * acc;
  }
}

template <typename TS, typename TQ>
static hipError_t scores_qjl_typed(const TQ* q, int64_t groups, int nq, const TS* S, int m,
                                   const uint32_t* bits, const uint16_t* norms, int64_t T, int d,
                                   float* scores, const DeviceInfo& dev, hipStream_t st) {
  const size_t lds = qjl_table_lds_floats(m) * sizeof(float);
  if (lds > dev.lds_per_block) return hipErrorInvalidConfiguration;
  // m = 256 with fp16 S and d <= 128: one workgroup per (group, tile) scores
  // all nq queries; else one per (group, query, tile)
  const bool grouped = m == 256 && sizeof(TS) == 2 && d <= 128;
  // one query: 1024-thread workgroups (8192-token tiles, one workgroup per
  // CU: one projection and one table build per CU) once the cache has more
  // than 4096 tokens, else 512; several: 512 threads once the cache fills
  // their tile (the queries' projections and table builds are then paid once
  // per 4096 tokens), else 256
  const int th = !grouped ? kQjlThreads
                 : nq == 1 ? (T > (int64_t)kQjlWideThreads * kQjlBatch ? kQjlOneQThreads
                                                                        : kQjlWideThreads)
                 : T >= (int64_t)kQjlWideThreads * kQjlBatch ? kQjlWideThreads
                                                             : kQjlThreads;
  const int64_t tile_tokens = grouped ? (int64_t)th * kQjlBatch : (int64_t)kQjlTok;
  const int64_t tiles = (T + tile_tokens - 1) / tile_tokens;
  const int64_t per_group = grouped ? tiles : tiles * nq;
  // launch in slices of whole groups so grid.x stays far below 2^32
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / per_group);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    const TQ* qp = q + g0 * nq * d;
    const uint32_t* bp = bits + g0 * T * (m / 32);
    const uint16_t* np = norms + g0 * T;
    float* sp = scores + g0 * nq * T;
    const unsigned blocks = (unsigned)(ng * per_group);
    auto launch = [&](auto kernel, int threads) {
      hipError_t e = allow_dynamic_lds(kernel, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kernel, dim3(blocks), dim3(threads), lds, st, qp, nq, S, m, d, bp, np, T,
                         tiles, sp);
      return hipGetLastError();
    };
    hipError_t e;
    if (grouped && nq == 1)
      e = th == kQjlOneQThreads
              ? launch(scores_qjl_kernel<TS, TQ, 8, kQjlOneQThreads, true>, th)
              : launch(scores_qjl_kernel<TS, TQ, 8, kQjlWideThreads, true>, th);
    else if (grouped)
      e = th == kQjlWideThreads ? launch(scores_qjl_kernel<TS, TQ, 8, kQjlWideThreads>, th)
                                : launch(scores_qjl_kernel<TS, TQ, 8>, th);
    else
      e = launch(scores_qjl_kernel<TS, TQ, 0>, kQjlThreads);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_scores_qjl(const void* q, int q_f16, int64_t groups, int nq, const void* S,
                             int S_f16, int m, const uint32_t* bits, const uint16_t* norms,
                             int64_t T, int d, float* scores, const DeviceInfo& dev,
                             hipStream_t st) {
  if (scores_qjl_gqa_supported(S_f16, m, d, nq) && scores_qjl_gqa_lds_bytes() <= dev.lds_per_block)
    return launch_scores_qjl_gqa(q, q_f16, groups, nq, static_cast<const _Float16*>(S), d, bits,
                                 norms, T, scores, dev, st);
  if (S_f16) {
    const _Float16* Sp = static_cast<const _Float16*>(S);
    if (q_f16)
      return scores_qjl_typed(static_cast<const _Float16*>(q), groups, nq, Sp, m, bits, norms, T, d,
                              scores, dev, st);
    return scores_qjl_typed(static_cast<const float*>(q), groups, nq, Sp, m, bits, norms, T, d,
                            scores, dev, st);
  }
  const float* Sp = static_cast<const float*>(S);
  if (q_f16)
    return scores_qjl_typed(static_cast<const _Float16*>(q), groups, nq, Sp, m, bits, norms, T, d,
                            scores, dev, st);
  return scores_qjl_typed(static_cast<const float*>(q), groups, nq, Sp, m, bits, norms, T, d,
                          scores, dev, st);
}

}  // namespace kvq
