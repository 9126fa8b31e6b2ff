// Device helpers shared by the QJL score and decode kernels.
#pragma once

#include "kvq_device.h"

namespace kvq {

constexpr float kSqrtHalfPi = 1.2533141373155001f;  // sqrt(pi / 2)

// Row of S that MFMA row i (0..31) of a 32-row tile reads.  The 32x32 MFMA
// result puts tile row i = 8q + 4h + s in accumulator register 4q + s of the
// lanes of half h; projection 16h + 4q + s is wanted there.
__host__ __device__ constexpr int sketch_row_perm(int i) {
  return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3);
}

// ---------------------------------------------------------------------------
// Query projection and byte tables (shared by the score and decode kernels).

// 16 values of type T from 16-byte-aligned memory, widened to binary32.
template <typename T>
__device__ __forceinline__ void load16_f32(const T* p, float out[16]);
template <>
__device__ __forceinline__ void load16_f32<float>(const float* p, float out[16]) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const f32x4 x = reinterpret_cast<const f32x4*>(p)[v];
    out[4 * v] = x[0]; out[4 * v + 1] = x[1]; out[4 * v + 2] = x[2]; out[4 * v + 3] = x[3];
  }
}
template <>
__device__ __forceinline__ void load16_f32<_Float16>(const _Float16* p, float out[16]) {
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    const f16x8 x = reinterpret_cast<const f16x8*>(p)[v];
#pragma unroll
    for (int e = 0; e < 8; ++e) out[8 * v + e] = (float)x[e];
  }
}

constexpr int kProjQChunk = 2048;   // query values staged in LDS per pass
constexpr int kProjMaxRowsPerThread = 4;

// a = fma chain of sr[j] * x[j] over j < len (len % 16 == 0) in j order, with
// the S loads of 64 channels issued together (one memory latency per 64
// channels instead of one per 16).  x is in LDS.
template <typename TS>
__device__ __forceinline__ float row_dot(const TS* __restrict__ sr, const float* x, int len,
                                         float a) {
  int j = 0;
  for (; j + 64 <= len; j += 64) {
    float sv[64];
#pragma unroll
    for (int c = 0; c < 4; ++c) load16_f32<TS>(sr + j + 16 * c, sv + 16 * c);
    const f32x4* xv = reinterpret_cast<const f32x4*>(x + j);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const f32x4 xx = xv[v];
      a = __builtin_fmaf(sv[4 * v + 0], xx[0], a);
      a = __builtin_fmaf(sv[4 * v + 1], xx[1], a);
      a = __builtin_fmaf(sv[4 * v + 2], xx[2], a);
      a = __builtin_fmaf(sv[4 * v + 3], xx[3], a);
    }
  }
  for (; j < len; j += 16) {
    float sv[16];
    load16_f32<TS>(sr + j, sv);
    const f32x4* xv = reinterpret_cast<const f32x4*>(x + j);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const f32x4 xx = xv[v];
      a = __builtin_fmaf(sv[4 * v + 0], xx[0], a);
      a = __builtin_fmaf(sv[4 * v + 1], xx[1], a);
      a = __builtin_fmaf(sv[4 * v + 2], xx[2], a);
      a = __builtin_fmaf(sv[4 * v + 3], xx[3], a);
    }
  }
  return a;
}

// y[i] = sum_j S[i][j] q[j] for i < m (m <= 1024), binary32 fused
// multiply-adds in j order, computed by the whole 256-thread workgroup:
// thread t owns rows t, t + 256, ...; q is staged through LDS (qs, at least
// kProjQChunk floats) and S rows are read 16 values at a time.
// y = S q for fp16 S with d <= 128 and m <= 64 * waves, coalesced: a wave
// load instruction reads 4 whole rows (16 lanes x 16 bytes each, 1 KiB
// contiguous); lane (row r4, chunk c) forms the 8 products of its chunk and
// the 16 lanes of a row are summed with DPP.  Two phases, so a caller can
// issue other loads between them: issue() requests the wave's rows of S and
// the thread's element of q (all unconditionally, so the compiler's wait
// counts stay exact), finish() stages q in LDS and writes y (callers
// synchronise before reading y).
// RG: row groups (4 rows each) held per wave, 16 covers m <= 64 * waves.
template <typename TQ, int RG = 16>
struct QueryProj16 {
  f16x8 raw[RG];
  TQ qreg;                          // converted in finish(), not here: a use
                                    // would make the compiler wait for the load
  int rpw;                          // rows per wave, a multiple of 4

  __device__ __forceinline__ static bool fits(int m, int d) {
    const int nw = (int)blockDim.x / 64;
    return d <= 128 && (int)blockDim.x >= d && ((m + nw - 1) / nw + 3) / 4 * 4 <= 4 * RG;
  }

  __device__ __forceinline__ void issue(const _Float16* __restrict__ S, const TQ* __restrict__ q,
                                        int m, int d) {
    const int nw = (int)blockDim.x / 64;
    rpw = ((m + nw - 1) / nw + 3) & ~3;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int r4 = lane >> 4;
    const int cc = min(c, d / 8 - 1);          // chunks past the row: reloaded, unused
#pragma unroll
    for (int it = 0; it < RG; ++it) {
      const int row = min(wave * rpw + 4 * min(it, rpw / 4 - 1) + r4, m - 1);
      raw[it] = *reinterpret_cast<const f16x8*>(S + (int64_t)row * d + 8 * cc);
    }
    qreg = q[min((int)threadIdx.x, d - 1)];
  }

  __device__ __forceinline__ void finish(float* qs, float* y, int m, int d) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = lane & 15;
    const int r4 = lane >> 4;
    const int cc = min(c, d / 8 - 1);
    // every thread writes (qs holds at least kProjQChunk >= blockDim.x floats;
    // entries past d are not read): a store under a branch would let the
    // compiler sink the q load next to it, behind the caller's later loads
    qs[threadIdx.x] = to_f32(qreg);
    __syncthreads();
    const bool live_c = 8 * c < d;
    float qv[8];
    const f32x4* p4 = reinterpret_cast<const f32x4*>(qs + 8 * cc);
    const f32x4 q0 = p4[0], q1 = p4[1];
    qv[0] = q0[0]; qv[1] = q0[1]; qv[2] = q0[2]; qv[3] = q0[3];
    qv[4] = q1[0]; qv[5] = q1[1]; qv[6] = q1[2]; qv[7] = q1[3];
    // all RG row groups are formed (past rpw they repeat the last one and are
    // not stored): a use under a branch would let the compiler sink the S
    // loads of issue() next to it
#pragma unroll
    for (int it = 0; it < RG; ++it) {
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)raw[it][e], qv[e], part);
      part = seg_sum_f32<16>(live_c ? part : 0.0f);
      const int row = wave * rpw + 4 * it + r4;
      if (c == 0 && 4 * it < rpw && row < m) y[row] = part;
    }
  }
};

// The same y = S q as QueryProj16 (same arithmetic, bit for bit) with only
// 4 row groups of S in registers at a time, for callers that hold many
// registers across it.  Starts with the q staging (the caller synchronises
// before, if qs is in use).
template <typename TQ>
__device__ __forceinline__ void project16_lite(const _Float16* __restrict__ S,
                                               const TQ* __restrict__ q, int m, int d, float* qs,
                                               float* y) {
  const int nw = (int)blockDim.x / 64;
  const int rpw = ((m + nw - 1) / nw + 3) & ~3;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int r4 = lane >> 4;
  const int cc = min(c, d / 8 - 1);
  qs[threadIdx.x] = to_f32(q[min((int)threadIdx.x, d - 1)]);
  __syncthreads();
  const bool live_c = 8 * c < d;
  float qv[8];
  const f32x4* p4 = reinterpret_cast<const f32x4*>(qs + 8 * cc);
  const f32x4 q0 = p4[0], q1 = p4[1];
  qv[0] = q0[0]; qv[1] = q0[1]; qv[2] = q0[2]; qv[3] = q0[3];
  qv[4] = q1[0]; qv[5] = q1[1]; qv[6] = q1[2]; qv[7] = q1[3];
  for (int it0 = 0; 4 * it0 < rpw; it0 += 4) {
    f16x8 raw[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = min(wave * rpw + 4 * min(it0 + k, rpw / 4 - 1) + r4, m - 1);
      raw[k] = *reinterpret_cast<const f16x8*>(S + (int64_t)row * d + 8 * cc);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float part = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) part = __builtin_fmaf((float)raw[k][e], qv[e], part);
      part = seg_sum_f32<16>(live_c ? part : 0.0f);
      const int row = wave * rpw + 4 * (it0 + k) + r4;
      if (c == 0 && 4 * (it0 + k) < rpw && row < m) y[row] = part;
    }
  }
}

template <typename TS, typename TQ>
__device__ __forceinline__ void project_query_block(const TS* __restrict__ S,
                                                    const TQ* __restrict__ q, int m, int d,
                                                    float* qs, float* y) {
  if constexpr (sizeof(TS) == 2) {
    if (QueryProj16<TQ>::fits(m, d)) {
      QueryProj16<TQ> pj;
      pj.issue(S, q, m, d);
      pj.finish(qs, y, m, d);
      return;
    }
  }
  float acc[kProjMaxRowsPerThread];
#pragma unroll
  for (int r = 0; r < kProjMaxRowsPerThread; ++r) acc[r] = 0.0f;
  for (int j0 = 0; j0 < d; j0 += kProjQChunk) {
    const int len = min(kProjQChunk, d - j0);
    __syncthreads();
    for (int j = threadIdx.x; j < len; j += blockDim.x) qs[j] = to_f32(q[j0 + j]);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kProjMaxRowsPerThread; ++r) {
      const int i = threadIdx.x + r * (int)blockDim.x;
      if (i < m) acc[r] = row_dot<TS>(S + (int64_t)i * d + j0, qs, len, acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < kProjMaxRowsPerThread; ++r) {
    const int i = threadIdx.x + r * (int)blockDim.x;
    if (i < m) y[i] = acc[r];
  }
}

// lut[p * 256 + v] = sum_{j<8} (bit j of v ? +1 : -1) * y[8p + j] for the
// nt = m / 8 tables, written as lo-nibble + hi-nibble partial sums.
__device__ void build_byte_tables(const float* y, int ntables, float* lut) {
  for (int task = threadIdx.x; task < ntables * 8; task += blockDim.x) {
    const int p = task >> 3;
    const int sub = task & 7;                  // entries v = 32 sub .. 32 sub + 31
    const float* yp = y + 8 * p;
    float lo[16];
    lo[0] = -(((yp[0] + yp[1]) + yp[2]) + yp[3]);
#pragma unroll
    for (int b = 1; b < 16; ++b) {
      const int low = b & (-b);
      const int j = __builtin_ctz(low);
      lo[b] = lo[b ^ low] + 2.0f * yp[j];
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int a = 2 * sub + hh;              // high nibble
      float hi = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) hi += ((a >> j) & 1) ? yp[4 + j] : -yp[4 + j];
#pragma unroll
      for (int b = 0; b < 16; ++b) lut[p * 256 + a * 16 + b] = hi + lo[b];
    }
  }
}

// ---------------------------------------------------------------------------
// Bank-conflict-free byte tables for m = 256 (32 tables, one per byte of a
// token's 256 sign bits).
//
// A lookup of the plain layout (lut[p * 256 + v]) by 64 lanes with random
// bytes v hits ~4 lanes per LDS bank.  Here row v (one per byte value, 64
// floats = 256 bytes, bank aligned) holds entry e = T_{e mod 32}[v], every
// table twice.  Lane L first rotates its 32 sign bytes by r = L mod 32, so at
// step i (0..31) it needs table (r + i) mod 32 and reads entry r + i of the
// row of its byte: the bank is (r + i) mod 64, different for every lane of a
// 32-lane half whatever the bytes are.  The lane's part of the address,
// 256 v + 4 r, is one byte permute; 4 i is the instruction's offset.
constexpr int kRotRowFloats = 64;
constexpr int kRotLutFloats = 256 * kRotRowFloats;

// Tables for projections of size m in floats, rotated layout or plain.
__host__ __device__ inline size_t byte_table_floats(int m, bool rotated) {
  return rotated ? (size_t)kRotLutFloats : (size_t)(m / 8) * 256;
}

// Rotated layout of the 32 tables of y[0..255]; entries hold the same
// binary32 values as build_byte_tables.
__device__ void build_rot_tables(const float* y, float* lut) {
  for (int task = threadIdx.x; task < 32 * 16; task += blockDim.x) {
    const int p = task & 31;                   // table
    const int a = task >> 5;                   // high nibble of v
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
    for (int b = 0; b < 16; ++b) {
      const float val = hi + lo[b];
      float* row = lut + (16 * a + b) * kRotRowFloats;
      row[p] = val;
      row[p + 32] = val;
    }
  }
}

// The 8 sign words of one token, as two 16-byte loads ordered by bit 4 of r
// (the first load starts at byte 16 * ((r >> 4) & 1)).
__device__ __forceinline__ void load_rot_words(const uint32_t* p, int r, uint32_t w[8]) {
  const int h = (r >> 4) & 1;
  const u32x4 a = ld_stream(reinterpret_cast<const u32x4*>(p + 4 * h));
  const u32x4 b = ld_stream(reinterpret_cast<const u32x4*>(p + 4 * (h ^ 1)));
  w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
  w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
}

typedef __attribute__((address_space(3))) const float* lds_cfloat_ptr;

// The lane's constant part of a rotated-table address: the tables' LDS
// address plus 4 r.  The byte permute below keeps bytes 0, 2 and 3 of it and
// puts the token's byte in byte 1, so the tables must start at an LDS address
// whose bits 8..15 are zero and whose low byte leaves room for 4 r (the
// kernels place them at the start of their LDS, address 0).
__device__ __forceinline__ uint32_t rot_lane_base(const float* lut, int r) {
  return (uint32_t)(uintptr_t)(lds_cfloat_ptr)lut + 4u * (uint32_t)r;
}

// The 8 words from load_rot_words rotated by the remaining 4 ((r >> 2) & 3)
// words and then r & 3 bytes, so that byte i of the result is byte (r + i)
// mod 32 of the token's sign bytes.  The word moves are bit blends with
// all-ones / all-zero lane masks (a select would become an indexed array in
// scratch).
__device__ __forceinline__ void rot_words(const uint32_t wl[8], int r, uint32_t x[8]) {
  uint32_t w[8];
  const uint32_t m2 = 0u - ((uint32_t)r >> 3 & 1u), m1 = 0u - ((uint32_t)r >> 2 & 1u);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = wl[j] ^ ((wl[(j + 2) & 7] ^ wl[j]) & m2);
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = x[j] ^ ((x[(j + 1) & 7] ^ x[j]) & m1);
  const uint32_t sh = 8u * (uint32_t)(r & 3);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_alignbit(w[(j + 1) & 7], w[j], sh);
}

// Sum over the 32 bytes of one token of the rotated tables' entries, for
// words already rotated by rot_words; rq is rot_lane_base(tables, r).
__device__ __forceinline__ float rot_lut_sum_rotated(const uint32_t x[8], uint32_t rq) {
  // Two halves of 16 reads, each kept in flight together (left to itself the
  // scheduler waits for each read before issuing the next); the sum is four
  // chains of 8 added pairwise.
  float part[4];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int i = 16 * hf + k;
      // LDS address: tables + (byte i & 3 of word i >> 2) * 256 + 4 r, + 4 i
      // as the instruction offset
      const uint32_t off =
          __builtin_amdgcn_perm(rq, x[i >> 2], 0x07060004u | ((uint32_t)(i & 3) << 8));
      v[k] = *(lds_cfloat_ptr)(uintptr_t)(off + 4u * (uint32_t)i);
    }
#pragma unroll
    for (int g = 0; g < 16; g += 8)
      asm volatile("" ::"v"(v[g]), "v"(v[g + 1]), "v"(v[g + 2]), "v"(v[g + 3]), "v"(v[g + 4]),
                   "v"(v[g + 5]), "v"(v[g + 6]), "v"(v[g + 7]));
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc += v[8 * c2 + k];
      part[2 * hf + c2] = acc;
    }
  }
  return (part[0] + part[1]) + (part[2] + part[3]);
}

// Sum over the 32 bytes of one token of the rotated tables' entries, for
// words loaded by load_rot_words with the same r (= lane % 32); rq is
// rot_lane_base(tables, r).
__device__ __forceinline__ float rot_lut_sum(const uint32_t wl[8], int r, uint32_t rq) {
  uint32_t x[8];
  rot_words(wl, r, x);
  return rot_lut_sum_rotated(x, rq);
}

// Sum of the table entries selected by the bytes of `nw` sign words.
__device__ __forceinline__ float lut_sum(const float* lut, const uint32_t* w, int nw) {
  float acc = 0.0f;
  for (int i = 0; i < nw; ++i) {
    const uint32_t x = w[i];
    const float* t = lut + i * 1024;
    acc += t[x & 0xFF];
    acc += t[256 + ((x >> 8) & 0xFF)];
    acc += t[512 + ((x >> 16) & 0xFF)];
    acc += t[768 + (x >> 24)];
  }
  return acc;
}

}  // namespace kvq
