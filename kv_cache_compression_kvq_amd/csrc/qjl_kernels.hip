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

#include <algorithm>
#include <cmath>

namespace kvq {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Sketch, fp16 keys on MFMA.  KS = d / 16 K-steps; MT = m / 32 projection
// tiles, a multiple of 8 (MT == 0: runtime m, words stored as they are
// produced).  Each wave
// owns NT x 32 tokens per iteration and loops over token tiles.
// Token tiles of 32 per wave iteration: two, or one when d = 256 would
// otherwise spill.
template <int KS> constexpr int sketch_nt() { return KS <= 8 ? 2 : 1; }
// Key tiles in flight per wave (a ring of register buffers).
template <int NT> constexpr int sketch_ring() { return NT == 1 ? 4 : 2; }

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

template <int KS, int MT>
__global__ __launch_bounds__(kSketchThreads) __attribute__((amdgpu_waves_per_eu(2)))
void sketch_mfma_kernel(const _Float16* __restrict__ k,
                                                          int64_t rows,
                                                          const _Float16* __restrict__ S,
                                                          int m_rt, uint32_t* __restrict__ bits,
                                                          uint16_t* __restrict__ norms) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  f16x8* sfrag = reinterpret_cast<f16x8*>(lds_raw);
  constexpr int D = KS * 16;
  const int mt_count = MT > 0 ? MT : m_rt / 32;
  const int words = mt_count;  // sign words per token
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  // S -> LDS in fragment order: fragment (mt, ks), lane l holds
  // S[32 mt + perm(l % 32)][16 ks + 8 (l / 32) .. + 8].
  const int nfrag_lanes = mt_count * KS * 64;
  for (int idx = tid; idx < nfrag_lanes; idx += kSketchThreads) {
    const int l = idx & 63;
    const int frag = idx >> 6;
    const int mt = frag / KS, ks = frag % KS;
    const int srow = 32 * mt + sketch_row_perm(l & 31);
    sfrag[idx] = *reinterpret_cast<const f16x8*>(S + (int64_t)srow * D + 16 * ks + 8 * (l >> 5));
  }
  __syncthreads();

  constexpr int kSketchNT = sketch_nt<KS>();
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
      if (h == 0 && tok < rows) norms[tok] = f32_to_f16_bits(__builtin_sqrtf(tot));
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
          if (h == 0 && tok < rows) bits[tok * words + mt] = f[nt];
        }
      }
    }
  };

  // RING token tiles in flight per wave: a ring of register buffers, each
  // refilled (unconditionally, clamped past the end) right after its tile's
  // multiplies are issued.
  constexpr int RING = sketch_ring<kSketchNT>();
  const int64_t stride = (int64_t)gridDim.x * kSketchWaves;
  const int64_t first = (int64_t)blockIdx.x * kSketchWaves + wave;
  if (first >= tiles) return;
  f16x8 bq[RING][kSketchNT][KS];
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
// Sketch, any shape (and fp32 keys): one thread per (row, sign word), 32
// binary32 dot products each; the word-0 thread also writes the norm.
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

template <int KS, int MT>
static hipError_t sketch_mfma_launch(const _Float16* k, int64_t rows, const _Float16* S, int m,
                                     uint32_t* bits, uint16_t* norms, const DeviceInfo& dev,
                                     hipStream_t st) {
  const size_t lds = (size_t)m * KS * 16 * sizeof(_Float16);
  constexpr int kSketchNT = sketch_nt<KS>();
  const int64_t tiles = (rows + 32 * kSketchNT - 1) / (32 * kSketchNT);
  // persistent grid: exactly the workgroups that fit on the device at once
  // (registers and LDS both limit it), each striding over the token tiles
  int per_cu = 0;
  hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, sketch_mfma_kernel<KS, MT>,
                                                              kSketchThreads, lds);
  if (e != hipSuccess) return e;
  const int64_t want = (tiles + kSketchWaves - 1) / kSketchWaves;
  const int64_t cap = (int64_t)dev.cus * std::max(1, per_cu);
  const int64_t blocks = std::max<int64_t>(1, std::min(want, cap));
  hipLaunchKernelGGL((sketch_mfma_kernel<KS, MT>), dim3((unsigned)blocks), dim3(kSketchThreads), lds, st, k,
                     rows, S, m, bits, norms);
  return hipGetLastError();
}

hipError_t launch_qjl_sketch(const void* k, int k_f16, int64_t rows, int d, const void* S, int m,
                             uint32_t* bits, uint16_t* norms, const DeviceInfo& dev,
                             hipStream_t st) {
  if (k_f16) {
    const size_t lds = (size_t)m * d * sizeof(_Float16);
    const _Float16* kh = static_cast<const _Float16*>(k);
    const _Float16* Sh = static_cast<const _Float16*>(S);
    if (lds <= std::min<size_t>(dev.lds_per_block, 64 * 1024)) {
      if (d == 128 && m == 256) return sketch_mfma_launch<8, 8>(kh, rows, Sh, m, bits, norms, dev, st);
      switch (d) {
        case 16: return sketch_mfma_launch<1, 0>(kh, rows, Sh, m, bits, norms, dev, st);
        case 32: return sketch_mfma_launch<2, 0>(kh, rows, Sh, m, bits, norms, dev, st);
        case 64: return sketch_mfma_launch<4, 0>(kh, rows, Sh, m, bits, norms, dev, st);
        case 128: return sketch_mfma_launch<8, 0>(kh, rows, Sh, m, bits, norms, dev, st);
        case 256: return sketch_mfma_launch<16, 0>(kh, rows, Sh, m, bits, norms, dev, st);
        default: break;
      }
    }
  }
  const int64_t threads = rows * (m / 32);
  const int64_t blocks = (threads + 255) / 256;
  // the generic path is launched in row slices to bound the grid
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
  (void)blocks;
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
constexpr int kQjlTokPerThread = 16;
constexpr int kQjlTok = kQjlThreads * kQjlTokPerThread;

// LDS: byte tables (rotated layout for m = 256, else [m / 8][256]) | y [m];
// the table area is also the query staging area of the projection, which
// ends before the tables are built.
__host__ __device__ inline size_t qjl_table_lds_floats(int m) {
  const size_t tables = byte_table_floats(m, m == 256);
  return (size_t)m + (tables > (size_t)kProjQChunk ? tables : (size_t)kProjQChunk);
}

// TH: threads per workgroup.  ONEQ: one query per group (the query loop is
// compiled out).  The m = 256 kernels stay under 128 registers so that two
// workgroups (64 KiB of tables each) share a CU at four waves per SIMD,
// which hides more of the lookups' LDS latency: the projection holds only
// four S rows at a time across the token loads, and per-lane token offsets
// are 32-bit from workgroup-uniform bases.
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
  // result plus the instruction offset, with no base to add
  float* lut = reinterpret_cast<float*>(lds_raw);
  const size_t tfl = byte_table_floats(m, m == 256);
  float* y = lut + (tfl > (size_t)kProjQChunk ? tfl : (size_t)kProjQChunk);
  const float c = kSqrtHalfPi / (float)m;
  if constexpr (W == 8) {
    constexpr int kTile = TH * kQjlBatch;
    // One workgroup per (group, tile) scores all nq queries of the group
    // (grouped-query attention: the queries of a KV head share one pass over
    // its sign words and norms, which stay in registers).  Per query: y = S q
    // and the byte tables are rebuilt in LDS, then the tokens are scored.
    // The tokens are requested before the first projection.  The loads are
    // unconditional (tokens past T re-read the tile's last token and are not
    // stored): loads under a branch make the compiler wait for each one.
    const int64_t g = blockIdx.x / tiles;
    const int64_t tile = blockIdx.x % tiles;
    const int64_t tbase = tile * kTile;
    const int nlive = (int)std::min<int64_t>(kTile, T - tbase);   // tokens of this tile
    const uint32_t* bg = bits + (g * T + tbase) * words;
    const uint16_t* ng = norms + g * T + tbase;
    const int r = threadIdx.x & 31;
    uint32_t wv[kQjlBatch][8];
    float nv[kQjlBatch];
    auto load_tokens = [&]() {
#pragma unroll
      for (int u = 0; u < kQjlBatch; ++u) {
        const int t = min((int)threadIdx.x + u * TH, nlive - 1);
        load_rot_words(bg + t * 8, r, wv[u]);
        nv[u] = (float)__builtin_bit_cast(_Float16, ld_stream(ng + t));
      }
    };
    // the words are rotated in place once (rot_words) and serve every query
    auto rotate_all = [&]() {
#pragma unroll
      for (int u = 0; u < kQjlBatch; ++u) {
        uint32_t xr[8];
        rot_words(wv[u], r, xr);
#pragma unroll
        for (int k = 0; k < 8; ++k) wv[u][k] = xr[k];
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
        const int t = (int)threadIdx.x + u * TH;
        const float acc = rot_lut_sum_rotated(wv[u], rq);
        if (t < nlive) st[t] = c * nv[u] * acc;
      }
    };
    // query 0 (this kernel is launched for fp16 S with d <= 128 only)
    const TQ* q0 = q + g * nq * d;
    if constexpr (sizeof(TS) == 2) {
      load_tokens();
      __builtin_amdgcn_sched_barrier(0);
      project16_lite(S, q0, m, d, lut, y);
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
  // one query: 512-thread workgroups, two per CU; several: 512 threads once
  // the cache fills their tile (the queries' projections and table builds
  // are then paid once per 4096 tokens), else 256
  const int th = !grouped ? kQjlThreads
                 : (nq == 1 || T >= (int64_t)kQjlWideThreads * kQjlBatch) ? kQjlWideThreads
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
      e = launch(scores_qjl_kernel<TS, TQ, 8, kQjlWideThreads, true>, kQjlWideThreads);
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
