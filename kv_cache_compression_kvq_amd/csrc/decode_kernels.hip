// One decode step of attention over a compressed cache for gfx950: keys as
// QJL sign sketches (arXiv 2406.03482, abstract: sign bits of a JL
// projection, scored against the unquantized projection of the query),
// values as per-row INT8 codes with a binary32 scale (symmetric INT8 formula
// of the Q-TensorFormer model card, section 6), consumed by softmax
// attention:
//   sigma_t = sqrt(pi/2)/m * n_t * sum_i (2 b_ti - 1) (S q)_i
//   out     = sum_t softmax_t(lam * sigma_t) * s_t * c_t
//
// Work split: the T tokens of a (batch, head) group are cut into `splits`
// ranges; one workgroup per (group, range, query) builds the byte tables from y = S q
// in LDS, streams its tokens once (sign words, norm, value codes, value
// scale) and keeps a running max / sum / weighted value sum per wave
// (online softmax).  The eight waves are merged in LDS and the workgroup
// writes (max, sum, o[d]) to the workspace; a second kernel merges the
// ranges with the log-sum-exp rule.  Nothing is materialised per token.
//
// Value codes are read 16 per lane (one 16-byte load) with LPV = d / 16
// lanes per token row, so a wave's load covers 64 / LPV whole rows (1 KiB);
// they are issued at the top of each 64-token chunk, before the scores that
// weight them are known, to keep HBM busy.
//
// Grouped-query attention (nq query heads per KV head): the nq workgroups of
// one (group, range) are numbered blockIdx = 8 (nq k + j) + x, so they run on
// the same XCD (workgroups go to XCD blockIdx mod 8) at about the same time
// and all but the first find the range's cache lines in that XCD's L2.
#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_qjl_device.h"

#include <algorithm>
#include <cmath>

namespace kvq {

constexpr int kDecodeWaves = 8;                        // waves per workgroup
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kDecodeChunk = 64;                       // tokens per wave step
constexpr int kDecodeBlockTokens = kDecodeWaves * kDecodeChunk;   // tokens per workgroup step

// DPP row rotate (lane i takes lane (i + n) % 16 of its 16-lane row).
template <int N>
__device__ __forceinline__ float dpp_ror_f32(float v) {
  return dpp_f32<0x120 + N>(v);
}

// Sum over the lanes that share lane % LPV (the `slot` bits above it).
template <int LPV>
__device__ __forceinline__ float slot_sum(float v) {
  if constexpr (LPV <= 4) v += dpp_ror_f32<4>(v);
  if constexpr (LPV <= 8) v += dpp_ror_f32<8>(v);
  if constexpr (LPV <= 16) v += swz_xor16_f32(v);
  if constexpr (LPV <= 32) v += xor32_f32(v);
  return v;
}

__device__ __forceinline__ float bcast_from(float v, int src_lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src_lane << 2, __builtin_bit_cast(int, v)));
}

// y[g] = S q[g] for every group, once per decode step (the split kernels of a
// group all read it from the workspace).
template <typename TS, typename TQ>
__global__ __launch_bounds__(256) void qjl_project_kernel(const TQ* __restrict__ q,
                                                          const TS* __restrict__ S, int m, int d,
                                                          float* __restrict__ y) {
  __shared__ __align__(16) float qs[kProjQChunk];
  const int64_t g = blockIdx.x;
  project_query_block(S, q + g * d, m, d, qs, y + g * m);
}

template <int W, int LPV>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(4))) void decode_split_kernel(
    const float* __restrict__ yall, int m_rt, int d, const uint32_t* __restrict__ kbits, const uint16_t* __restrict__ knorms,
    const int8_t* __restrict__ vcodes, const float* __restrict__ vscales, int64_t T,
    int64_t splits, int64_t tps, float lam, int nq, int64_t pairs, float* __restrict__ partials) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int m = W > 0 ? 32 * W : m_rt;
  const int words = m / 32;
  // tables first: at LDS address 0 a lookup's address needs no base added
  float* lut = reinterpret_cast<float*>(lds_raw);
  float* y = lut + byte_table_floats(m, W == 8);
  float* wpart = y + m;                                // [kDecodeWaves][d + 2]

  // (group, range) pair p and query j of this workgroup; padding workgroups
  // past the last pair exit here, before any barrier
  const int64_t bx = blockIdx.x;
  const int64_t rest = bx >> 3;
  const int jq = (int)(rest % nq);
  const int64_t p = (rest / nq) * 8 + (bx & 7);
  if (p >= pairs) return;
  const int64_t g = p / splits;             // KV group
  const int64_t sp = p % splits;
  const int64_t vg = g * nq + jq;           // query (group, head)
  const int64_t t_begin = sp * tps;
  const int64_t t_end = std::min<int64_t>(T, t_begin + tps);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  constexpr int SLOTS = kWave / LPV;      // value rows per wave load
  constexpr int VSTEPS = kDecodeChunk / SLOTS;
  constexpr bool PREFETCH = LPV <= 16;
  constexpr int DV = PREFETCH ? 16 * LPV : 0;   // compile-time d when LPV fixes it
  const int dd = DV > 0 ? DV : d;
  const int sub = lane % LPV;
  const int slot = lane / LPV;
  const int cpr = dd / 16;                 // 16-code chunks per value row
  const bool sub_live = sub < cpr;         // LPV == 64 covers d < 1024 with idle lanes
  const float c = kSqrtHalfPi / (float)m;
  // Per-workgroup bases; everything below is a 32-bit offset from them (a
  // token range holds at most 2^31 / (d + m / 8) tokens, checked on launch).
  const int64_t row0 = g * T + t_begin;
  const uint32_t* bblk = kbits + row0 * words;
  const uint16_t* nblk = knorms + row0;
  const int8_t* vblk = vcodes + row0 * dd + sub * 16;
  const float* sblk = vscales + row0;
  const int ntok = (int)(t_end - t_begin);

  float M = -INFINITY, L = 0.0f;
  float o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.0f;

  if constexpr (W == 8 && PREFETCH) {
    // Software pipeline over the wave's 64-token chunks: the loads of the
    // next chunk (value codes, sign words, norm, value scale) are issued
    // before the current chunk is scored and accumulated, and the first
    // chunk's before the byte tables are built.  Every load is unconditional
    // (past the range: the last token, weight 0), so the compiler's wait
    // counts leave the next chunk in flight.
    // Sign words, norm and value scale of a chunk (needed first, for the
    // scores) and its value codes (needed last) are loaded separately, so
    // the next chunk's value codes are requested only once the current
    // chunk's score temporaries are dead.
    struct Keys {
      uint32_t wv[8];
      uint16_t nb;
      float vs;
    };
    struct Vals {
      u32x4 vc[VSTEPS];
    };
    const int r = lane & 31;
    auto load_keys = [&](Keys& kk, int base) {
      const int tc = min(base + lane, ntok - 1);
      load_rot_words(bblk + tc * 8, r, kk.wv);
      kk.nb = ld_stream(nblk + tc);
      kk.vs = ld_stream(sblk + tc);
    };
    auto load_vals = [&](Vals& vv, int base) {
#pragma unroll
      for (int i = 0; i < VSTEPS; ++i) {
        const int tv = min(base + i * SLOTS + slot, ntok - 1);
        vv.vc[i] = ld_stream(reinterpret_cast<const u32x4*>(vblk + tv * DV));
      }
    };
    // softmax weight times value scale of this lane's token
    auto score = [&](const Keys& kk, int base) -> float {
      const bool valid = base + lane < ntok;
      const float acc = rot_lut_sum(kk.wv, r, rot_lane_base(lut, r));
      const float n = (float)__builtin_bit_cast(_Float16, kk.nb);
      const float z = valid ? lam * (c * n * acc) : -INFINITY;
      // online softmax update (lane 0 of every chunk is valid, so mx is finite)
      const float mx = seg_max_f32<64>(z);
      const float M_new = __builtin_fmaxf(M, mx);
      const float alpha = __expf(M - M_new);        // 0 on the first chunk (M = -inf)
      const float p = __expf(z - M_new);            // 0 for invalid tokens (z = -inf)
      L = L * alpha + seg_sum_f32<64>(p);
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] *= alpha;
      M = M_new;
      return p * kk.vs;
    };
    auto accumulate = [&](const Vals& vv, float ps) {
#pragma unroll
      for (int i = 0; i < VSTEPS; ++i) {
        const float w = bcast_from(ps, i * SLOTS + slot);
#pragma unroll
        for (int e = 0; e < 16; ++e)
          o[e] = __builtin_fmaf(w, i8_to_f32(vv.vc[i][e >> 2], e & 3), o[e]);
      }
    };

    // y first (so its wait leaves the chunk loads in flight); every thread
    // writes, past m into the merge area, which is written again later
    const float yv = yall[vg * m + min((int)threadIdx.x, m - 1)];
    const int first = wave * kDecodeChunk;
    Keys ka, kb;
    Vals va, vb;
    __builtin_amdgcn_sched_barrier(0);
    load_keys(ka, first);
    load_vals(va, first);
    __builtin_amdgcn_sched_barrier(0);
    y[threadIdx.x] = yv;
    __syncthreads();
    build_rot_tables(y, lut);
    __syncthreads();
    if (first < ntok) {
      for (int base = first;; base += 2 * kDecodeBlockTokens) {
        const int nb1 = base + kDecodeBlockTokens, nb2 = base + 2 * kDecodeBlockTokens;
        load_keys(kb, nb1);
        const float psa = score(ka, base);
        accumulate(va, psa);
        load_vals(vb, nb1);
        if (nb1 >= ntok) break;
        load_keys(ka, nb2);
        const float psb = score(kb, nb1);
        accumulate(vb, psb);
        load_vals(va, nb2);
        if (nb2 >= ntok) break;
      }
    }
  } else {
    for (int i = threadIdx.x; i < m; i += kDecodeThreads) y[i] = yall[vg * m + i];
    __syncthreads();
    build_byte_tables(y, m / 8, lut);
    __syncthreads();
    for (int base = wave * kDecodeChunk; base < ntok; base += kDecodeBlockTokens) {
      // Tokens past the range are clamped to its last token: their loads stay
      // in bounds and their softmax weight is forced to 0 below.
      const int t = base + lane;
      const bool valid = t < ntok;
      const int tc = min(t, ntok - 1);
      u32x4 vc[PREFETCH ? VSTEPS : 1];
      if constexpr (PREFETCH) {
  #pragma unroll
        for (int i = 0; i < VSTEPS; ++i) {
          const int tv = min(base + i * SLOTS + slot, ntok - 1);
          vc[i] = ld_stream(reinterpret_cast<const u32x4*>(vblk + tv * DV));
        }
      }
      float acc = 0.0f;
      for (int i = 0; i < words; ++i) {
        const uint32_t x = bblk[tc * words + i];
        acc += lut_sum(lut + i * 1024, &x, 1);
      }
      const float n = (float)__builtin_bit_cast(_Float16, ld_stream(nblk + tc));
      const float vs = ld_stream(sblk + tc);
      const float z = valid ? lam * (c * n * acc) : -INFINITY;
      // online softmax update (lane 0 of every chunk is valid, so mx is finite)
      const float mx = seg_max_f32<64>(z);
      const float M_new = __builtin_fmaxf(M, mx);
      const float alpha = __expf(M - M_new);        // 0 on the first chunk (M = -inf)
      const float p = __expf(z - M_new);            // 0 for invalid tokens (z = -inf)
      L = L * alpha + seg_sum_f32<64>(p);
  #pragma unroll
      for (int e = 0; e < 16; ++e) o[e] *= alpha;
      M = M_new;
      const float ps = p * vs;
      // o += p_t * s_t * c_t over the chunk's value rows
      if constexpr (PREFETCH) {
  #pragma unroll
        for (int i = 0; i < VSTEPS; ++i) {
          const float w = bcast_from(ps, i * SLOTS + slot);
  #pragma unroll
          for (int e = 0; e < 16; ++e) o[e] = __builtin_fmaf(w, i8_to_f32(vc[i][e >> 2], e & 3), o[e]);
        }
      } else {
        for (int i = 0; i < VSTEPS; ++i) {
          const float w = bcast_from(ps, i * SLOTS + slot);
          const int tv = min(base + i * SLOTS + slot, ntok - 1);
          const u32x4 cw = sub_live ? *reinterpret_cast<const u32x4*>(vblk + tv * dd) : u32x4{};
  #pragma unroll
          for (int e = 0; e < 16; ++e) o[e] = __builtin_fmaf(w, i8_to_f32(cw[e >> 2], e & 3), o[e]);
        }
      }
    }
  }

  // merge the slots of the wave, then the four waves of the workgroup
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = slot_sum<LPV>(o[e]);
  float* wp = wpart + wave * (d + 2);
  if (lane == 0) {
    wp[0] = M;
    wp[1] = L;
  }
  if (slot == 0 && sub_live) {
#pragma unroll
    for (int e = 0; e < 16; ++e) wp[2 + sub * 16 + e] = o[e];
  }
  __syncthreads();
  float Mw[kDecodeWaves], Ms = -INFINITY;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) {
    Mw[w] = wpart[w * (d + 2)];
    Ms = __builtin_fmaxf(Ms, Mw[w]);
  }
  float sc[kDecodeWaves];
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) sc[w] = (Mw[w] == -INFINITY) ? 0.0f : __expf(Mw[w] - Ms);
  float* out = partials + (vg * splits + sp) * (int64_t)(d + 2);
  if (threadIdx.x == 0) {
    float Ls = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) Ls += sc[w] * wpart[w * (d + 2) + 1];
    out[0] = Ms;
    out[1] = Ls;
  }
  for (int j = threadIdx.x; j < d; j += kDecodeThreads) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w)
      if (sc[w] != 0.0f) acc += sc[w] * wpart[w * (d + 2) + 2 + j];
    out[2 + j] = acc;
  }
}

// out[g, j] = sum_k e^{M_k - M} o_k[j] / sum_k e^{M_k - M} L_k over the splits.
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ partials,
                                                           int64_t groups, int64_t splits, int d,
                                                           float* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= groups * d) return;
  const int64_t g = idx / d;
  const int j = (int)(idx % d);
  const float* pg = partials + g * splits * (int64_t)(d + 2);
  float Ms = -INFINITY;
  for (int64_t k = 0; k < splits; ++k) Ms = __builtin_fmaxf(Ms, pg[k * (d + 2)]);
  float num = 0.0f, den = 0.0f;
  for (int64_t k = 0; k < splits; ++k) {
    const float Mk = pg[k * (d + 2)];
    if (Mk == -INFINITY) continue;
    const float wgt = __expf(Mk - Ms);
    den += wgt * pg[k * (d + 2) + 1];
    num += wgt * pg[k * (d + 2) + 2 + j];
  }
  out[idx] = num / den;
}

DecodeSplit decode_split(int64_t groups, int64_t T, const DeviceInfo& dev) {
  DecodeSplit s;
  // about 8 workgroups per CU in all (four rounds of the two that fit at
  // once): at 512 query groups x 32768 tokens, 4 ranges per group measured
  // 2-3 % faster than 3 or 8 (the last round's tail and the per-workgroup
  // table build against the number of rounds)
  const int64_t target_blocks = 8LL * std::max(1, dev.cus);
  const int64_t max_splits = std::max<int64_t>(1, (T + kDecodeBlockTokens - 1) / kDecodeBlockTokens);
  int64_t splits = std::min(max_splits, std::max<int64_t>(1, (target_blocks + groups - 1) / groups));
  // token ranges of at most 2^20 tokens keep every in-kernel offset in 32 bits
  splits = std::max<int64_t>(splits, (T + (int64_t(1) << 20) - 1) >> 20);
  int64_t tps = (T + splits - 1) / splits;
  tps = (tps + kDecodeBlockTokens - 1) / kDecodeBlockTokens * kDecodeBlockTokens;
  s.tokens_per_split = tps;
  s.splits = (T + tps - 1) / tps;
  return s;
}

// Workspace: y [groups][m] (padded to 256 B), then partials [groups][splits][d + 2].
static size_t decode_y_bytes(int64_t groups, int m) {
  return ((size_t)groups * (size_t)m * sizeof(float) + 255) / 256 * 256;
}

// Token split of a call: the one-pass grouped kernel's for several queries
// per KV head where it applies, else the one-query kernel's over all queries.
static DecodeSplit call_split(int64_t groups, int nq, int64_t T, int d, int m,
                              const DeviceInfo& dev) {
  return decode_gqa_supported(m, d, nq) ? decode_gqa_split(groups, T, dev)
                                        : decode_split(groups * nq, T, dev);
}

size_t decode_workspace_bytes(int64_t groups, int nq, int64_t T, int d, int m,
                              const DeviceInfo& dev) {
  const DecodeSplit s = call_split(groups, nq, T, d, m, dev);
  return decode_y_bytes(groups * nq, m) +
         (size_t)groups * (size_t)nq * (size_t)s.splits * (size_t)(d + 2) * sizeof(float);
}

// The specialised kernel (m = 256, d = 128) reads the rotated byte tables.
static bool decode_rotated(int m, int d) { return m == 256 && d == 128; }

size_t decode_lds_bytes(int m, int d) {
  return ((size_t)m + byte_table_floats(m, decode_rotated(m, d)) + kDecodeWaves * (size_t)(d + 2)) *
         sizeof(float);
}

template <int W, int LPV>
static hipError_t decode_launch(const float* y, int64_t groups, int nq, int m,
                                const uint32_t* kbits, const uint16_t* knorms,
                                const int8_t* vcodes, const float* vscales, int64_t T, int d,
                                float lam, float* partials, const DecodeSplit& sp,
                                hipStream_t st) {
  const size_t lds = decode_lds_bytes(m, d);
  hipError_t e0 = allow_dynamic_lds(decode_split_kernel<W, LPV>, lds);
  if (e0 != hipSuccess) return e0;
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 21) / (sp.splits * nq));
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, groups - g0);
    const int64_t pairs = ng * sp.splits;
    const int64_t blocks = (pairs + 7) / 8 * 8 * nq;
    hipLaunchKernelGGL((decode_split_kernel<W, LPV>), dim3((unsigned)blocks),
                       dim3(kDecodeThreads), lds, st, y + g0 * nq * m, m, d,
                       kbits + g0 * T * (m / 32), knorms + g0 * T, vcodes + g0 * T * d,
                       vscales + g0 * T, T, sp.splits, sp.tokens_per_split, lam, nq, pairs,
                       partials + g0 * nq * sp.splits * (d + 2));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename TS, typename TQ>
static hipError_t decode_typed(const TQ* q, int64_t groups, int nq, const TS* S, int m,
                               const uint32_t* kbits, const uint16_t* knorms, const int8_t* vcodes,
                               const float* vscales, int64_t T, int d, float lam, void* ws,
                               float* out, const DeviceInfo& dev, hipStream_t st) {
  // queries are numbered (group, head) = g nq + j throughout: y, partials, out
  const int64_t nqg = groups * nq;
  const DecodeSplit sp = call_split(groups, nq, T, d, m, dev);
  float* y = static_cast<float*>(ws);
  float* partials = reinterpret_cast<float*>(static_cast<char*>(ws) + decode_y_bytes(nqg, m));
  const int64_t max_groups = int64_t(1) << 22;
  for (int64_t g0 = 0; g0 < nqg; g0 += max_groups) {
    const int64_t ng = std::min(max_groups, nqg - g0);
    hipLaunchKernelGGL((qjl_project_kernel<TS, TQ>), dim3((unsigned)ng), dim3(256), 0, st,
                       q + g0 * d, S, m, d, y + g0 * m);
    hipError_t e1 = hipGetLastError();
    if (e1 != hipSuccess) return e1;
  }
  hipError_t e = hipSuccess;
  if (decode_gqa_supported(m, d, nq)) {
    // one pass over each token range per four query heads
    for (int q0 = 0; q0 < nq && e == hipSuccess; q0 += 4)
      e = launch_decode_gqa_pass(y, groups, nq, q0, std::min(4, nq - q0), kbits, knorms, vcodes,
                                 vscales, T, lam, partials, sp, st);
  } else if (decode_rotated(m, d))
    e = decode_launch<8, 8>(y, groups, nq, m, kbits, knorms, vcodes, vscales, T, d, lam, partials, sp, st);
  else if (d == 64)
    e = decode_launch<0, 4>(y, groups, nq, m, kbits, knorms, vcodes, vscales, T, d, lam, partials, sp, st);
  else if (d == 128)
    e = decode_launch<0, 8>(y, groups, nq, m, kbits, knorms, vcodes, vscales, T, d, lam, partials, sp, st);
  else if (d == 256)
    e = decode_launch<0, 16>(y, groups, nq, m, kbits, knorms, vcodes, vscales, T, d, lam, partials, sp, st);
  else
    e = decode_launch<0, 64>(y, groups, nq, m, kbits, knorms, vcodes, vscales, T, d, lam, partials, sp, st);
  if (e != hipSuccess) return e;
  const int64_t n = nqg * d;
  hipLaunchKernelGGL(decode_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     partials, nqg, sp.splits, d, out);
  return hipGetLastError();
}

hipError_t launch_decode_qjl_int8(const void* q, int q_f16, int64_t groups, int nq, const void* S,
                                  int S_f16, int m, const uint32_t* kbits, const uint16_t* knorms,
                                  const int8_t* vcodes, const float* vscales, int64_t T, int d,
                                  float sm_scale, void* ws, float* out, const DeviceInfo& dev,
                                  hipStream_t st) {
  if (S_f16) {
    const _Float16* Sp = static_cast<const _Float16*>(S);
    if (q_f16)
      return decode_typed(static_cast<const _Float16*>(q), groups, nq, Sp, m, kbits, knorms, vcodes,
                          vscales, T, d, sm_scale, ws, out, dev, st);
    return decode_typed(static_cast<const float*>(q), groups, nq, Sp, m, kbits, knorms, vcodes,
                        vscales, T, d, sm_scale, ws, out, dev, st);
  }
  const float* Sp = static_cast<const float*>(S);
  if (q_f16)
    return decode_typed(static_cast<const _Float16*>(q), groups, nq, Sp, m, kbits, knorms, vcodes,
                        vscales, T, d, sm_scale, ws, out, dev, st);
  return decode_typed(static_cast<const float*>(q), groups, nq, Sp, m, kbits, knorms, vcodes, vscales,
                      T, d, sm_scale, ws, out, dev, st);
}

}  // namespace kvq
