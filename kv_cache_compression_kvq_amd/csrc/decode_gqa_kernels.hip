// Grouped-query decode in one pass over the cache, for gfx950: nq query heads
// share each KV head's compressed keys and values (the Q-TensorFormer model
// card, section 4, shares a KV head among several query heads).  Per query
// the step is the decode of one query over QJL-sketched keys (arXiv
// 2406.03482, abstract: sign bits of a JL projection, scored against the
// query's unquantized projection) and per-row INT8 values (symmetric INT8
// formula of the same card, section 6):
//   sigma_t = sqrt(pi/2)/m * n_t * sum_i (2 b_ti - 1) (S q)_i
//   out     = sum_t softmax_t(lam * sigma_t) * s_t * c_t
// Here one workgroup per (KV head, token range) reads the range once and
// carries up to four of the head's queries through it: the scores of each
// 32-token wave step on the matrix cores (below), four online softmaxes,
// the four weighted value sums on the matrix cores from each value load.
// Heads with more queries take one launch per four.
//
// Scores, on the matrix cores: for a tile of 16 tokens, sum_i (2 b_ti - 1)
// y_i for every query is the product of the tokens' +-1 sign matrix
// (16 x 256) and the queries' projections (256 x NQ): the signs reach the A
// operand through an LDS table of the 256 byte values' +-1 expansions, the
// projections are the B operand as binary16 hi / lo parts (column j the hi
// part of query j, column j + 8 its lo part, after a power-of-two scaling
// per query), eight v_mfma_f32_16x16x32_f16 per tile.  The step's sums go
// through a few LDS floats of the wave so that lane (r, h) = (lane % 32,
// lane / 32) receives token r's score for query 2 b + h (b < NQ / 2), the
// layout of the softmax below.  (The byte-table lookups used before cost
// 32 per token and query, which bound the kernel by vector-ALU issue.)

// Values, on the matrix cores: per wave step, o[q][ch] += sum over the 32
// tokens of w[q][t] c[t][ch] is eight v_mfma_f32_16x16x32_f16 (one per group
// of 16 channels), the weights w = softmax weight x value scale as the A
// operand (rows: the queries' binary16 hi halves, then their lo halves) and
// the codes as the B operand (int8 -> binary16 exactly).  The contraction
// runs over tokens, so lane (nl, kq) = (lane % 16, lane / 16) loads 8 bytes
// (channels 8 nl .. 8 nl + 7) of each of the tokens 8 kq .. 8 kq + 7 (whole
// rows per load instruction) and column nl of group j is channel 8 nl + j.
// The weights reach the A fragments through 512 B of LDS per wave; they are
// scaled by 2^(14 - R), R the exponent of the largest value scale the wave
// has seen, so they stay within binary16's range (the sums are rescaled
// with the softmax's own factor when R grows).  Partials (max, sum, o[d]) per
// (query, token range) go to the same workspace layout as the one-query
// decode, whose merge kernel finishes the step.
#include "kvq_device.h"
#include "kvq_launch.h"
#include "kvq_qjl_device.h"
#include "kvq_qjl_stream.h"

#include <algorithm>
#include <cmath>

namespace kvq {

constexpr int kGqaChunk = 32;                            // tokens per wave step
// waves per workgroup: the four-query kernel takes 12 (one workgroup per
// CU, 3 waves per SIMD), the two-query kernel two 8-wave workgroups per CU
constexpr int gqa_waves(int nb) { return nb == 2 ? 12 : 8; }
constexpr int kGqaBlockTokens = 8 * kGqaChunk;           // token-range granule
constexpr int kGqaD = 128, kGqaM = 256;

// --- signs on the matrix cores (shared by the decode and the scores) --------
//
// A operand from sign bytes: lane (t, kq) = (lane % 16, lane / 16) holds
// bytes 8 kq .. 8 kq + 7 of token t's 32-byte sign row and, at K-step ks,
// reads the 16-byte +-1 expansion of byte 8 kq + ks (bit e -> element e,
// binary16 +1 / -1) from an LDS table that holds one copy per lane position
// t: entry (v, t) at 256 v + 16 t, so the 16 lanes of each group read 16
// different bank quads whatever the bytes.  The address is one byte permute
// (the byte into byte 1, 16 t in byte 0): the table sits at LDS address 0,
// and the kernels using it declare no static __shared__ data.  MFMA row t,
// K index 32 ks + 8 kq + e is then projection 8 (8 kq + ks) + e =
// 64 kq + 8 ks + e, where the B operand holds the projections.
constexpr uint32_t kSignTableBytes = 256u * 16u * 16u;         // 64 KiB
typedef __attribute__((address_space(3))) const f16x8* lds_cf16x8_ptr;
__device__ __forceinline__ void build_sign_table(unsigned char* lds, int tid, int nthreads) {
  for (int i = tid; i < 256 * 16; i += nthreads) {
    const uint32_t v = (uint32_t)i >> 4;
    u32x4 ent;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      ent[w] = (((v >> (2 * w)) & 1u) ? 0x3C00u : 0xBC00u) |
               ((((v >> (2 * w + 1)) & 1u) ? 0x3C00u : 0xBC00u) << 16);
    *reinterpret_cast<u32x4*>(lds + 16 * i) = ent;
  }
}

// Expansion of byte ks (0..7) of the lane's 8 sign bytes w; tbyte = 16 t.
__device__ __forceinline__ f16x8 sign_fragment(const u32x2& w, int ks, uint32_t tbyte) {
  const uint32_t a = __builtin_amdgcn_perm(w[ks >> 2], tbyte, 0x0C0C0000u | ((4u + (uint32_t)(ks & 3)) << 8));
  return *(lds_cf16x8_ptr)(uintptr_t)a;
}

// 2^(14 - e), e the exponent of the largest magnitude (its binary32 bits
// without the sign); the scaled vector's largest magnitude lies in
// [2^14, 2^15).
__device__ __forceinline__ float gm_pow2_scale(uint32_t max_abs_bits) {
  const int e = max_abs_bits == 0 ? 0 : (int)((max_abs_bits >> 23) & 0xFF) - 127;
  return __builtin_ldexpf(1.0f, min(14 - e, 126));
}

// hi = v with its 13 low significand bits cleared, lo = v - hi (exact in
// binary32) rounded toward zero, both binary16: hi + lo is within 2^-21 of
// v, relative (2^-24 absolute below binary16's normal range).
__device__ __forceinline__ void gm_split(float v, _Float16& hi, _Float16& lo) {
  const float h = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xFFFFE000u);
  const auto p = __builtin_amdgcn_cvt_pkrtz(h, v - h);
  hi = p[0];
  lo = p[1];
}

// The value of lane ^ 8 (DPP row_ror:8 inside each 16-lane row).
__device__ __forceinline__ float gm_xor8(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, true));
}

constexpr int kGqaYs = kGqaM + 8;    // padded row of a projection in LDS

// NQ = 2 NB query slots per launch.  yall: projected queries
// [groups * nq_total][m]; this launch takes queries q_off .. q_off + nq_pass
// - 1 of every group (nq_pass <= 2 NB; the other slots score against a zero
// projection and are not written).
template <int NB, int WAVES = gqa_waves(NB)>
// (eight-wave workgroups run two per CU: at most 128 registers)
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES == 8 ? 4 : WAVES / 4)))
void decode_gqa_kernel(const float* __restrict__ yall, int nq_total, int q_off, int nq_pass,
                       const uint32_t* __restrict__ kbits, const uint16_t* __restrict__ knorms,
                       const int8_t* __restrict__ vcodes, const float* __restrict__ vscales,
                       int64_t T, int64_t splits, int64_t tps, float lam, int64_t pairs,
                       float* __restrict__ partials) {
  constexpr int NQ = 2 * NB;
  constexpr int D = kGqaD, M = kGqaM;
  extern __shared__ __align__(16) unsigned char lds_raw[];
  // the sign table first, at LDS address 0 (no static __shared__ data here)
  float* y = reinterpret_cast<float*>(lds_raw + kSignTableBytes);        // [NQ][kGqaYs]
  float* yscale = y + NQ * kGqaYs;                                        // [4]
  f16x8* byf = reinterpret_cast<f16x8*>(yscale + 4);                      // [8][64]
  float* wpart = reinterpret_cast<float*>(lds_raw);   // [waves][NQ][D + 2], after the last lookup

  const int64_t p = blockIdx.x;
  if (p >= pairs) return;
  const int64_t g = p / splits;
  const int64_t sp = p % splits;
  const int64_t t_begin = sp * tps;
  const int ntok = (int)(std::min<int64_t>(T, t_begin + tps) - t_begin);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 31;                   // token of the wave step (scoring)
  const int h = lane >> 5;                   // query slot within each block
  const int nl = lane & 15;                  // matrix-core row / column of the lane
  const int kq = lane >> 4;                  // its 8-token group of the step
  const float c = kSqrtHalfPi / (float)M;
  const int64_t row0 = g * T + t_begin;
  const uint32_t* bblk = kbits + row0 * (M / 32);
  const uint16_t* nblk = knorms + row0;
  const int8_t* vblk = vcodes + row0 * D + 8 * nl;
  const float* sblk = vscales + row0;
  // per wave: the step's softmax weights [NQ][32], staged for the matrix
  // cores, and its scores [NQ][32], staged for the softmax
  float* wst = reinterpret_cast<float*>(byf + 8 * 64) + wave * NQ * kGqaChunk;
  float* zs = reinterpret_cast<float*>(byf + 8 * 64) + (WAVES + wave) * NQ * kGqaChunk;
  int* next_step = reinterpret_cast<int*>(byf + 8 * 64) + 2 * WAVES * NQ * kGqaChunk;   // steps handed out

  struct Keys {
    u32x2 w[2];                              // sign bytes 8 kq .. + 7 of token 16 u + nl
    uint16_t nb;                             // norm of token r
    float vs;                                // value scale of token r
  };
  struct Vals {
    u32x2 vc[8];                             // channels 8 nl .. + 7 of tokens 8 kq + e
  };
  // the step's sign words: each load instruction reads a tile's 16 rows
  auto load_keys = [&](Keys& kk, int base) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int tk = min(base + 16 * u + nl, ntok - 1);
      kk.w[u] = ld_stream(reinterpret_cast<const u32x2*>(bblk + tk * 8 + 2 * kq));
    }
    const int tc = min(base + r, ntok - 1);
    kk.nb = ld_stream(nblk + tc);
    kk.vs = ld_stream(sblk + tc);
  };
  // whole rows per instruction: 4 tokens x 16 lanes x 8 B
  auto load_vals = [&](Vals& vv, int base) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tv = min(base + 8 * kq + e, ntok - 1);
      vv.vc[e] = ld_stream(reinterpret_cast<const u32x2*>(vblk + tv * D));
    }
  };

  // B fragments of the scores (column j < NQ: query j's hi part, j + 8 its
  // lo part, other columns zero), set up below
  f16x8 by[8];
  float yunscale = 1.0f;
  const uint32_t tbyte = 16u * (uint32_t)nl;

  // value sums on the matrix cores: acc[j] = D tile of channel group j,
  // row rho = (part, query) = (rho / NQ, rho % NQ) with part 0 the weights'
  // hi halves, part 1 their lo halves (rows past 2 NQ stay zero), column nl
  // = channel 8 nl + j; lane (nl, kq) holds rows 4 kq .. 4 kq + 3
  // Mq: running maxima (per query, the same in every lane); Ll: this lane's
  // share of the softmax denominators (its tokens, query 2 b + h), summed
  // over the lanes once at the end
  float Mq[NQ], Ll[NB];
  f32x4 acc[8];
#pragma unroll
  for (int q = 0; q < NQ; ++q) Mq[q] = -INFINITY;
#pragma unroll
  for (int b = 0; b < NB; ++b) Ll[b] = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // weights are scaled by 2^(14 - R), R the exponent of the largest value
  // scale seen so far by the wave (a softmax weight is at most 1), so the
  // largest lies below 2^15 and binary16 keeps 22 bits of each through its
  // hi / lo split; R only grows, and the sums are rescaled when it does
  int R = -110;

  // z of this lane's token r for query 2 b + h (-inf past the range): the
  // step's two 16-token tiles on the matrix cores, their sums handed to the
  // softmax layout through the wave's LDS rows zs (LDS operations of one
  // wave complete in order; the asm statements keep the compiler from
  // moving them across each other)
  auto scores = [&](const Keys& kk, int base, float (&z)[NB]) {
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f16x8 sg[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sg[ks] = sign_fragment(kk.w[u], ks, tbyte);
      f32x4 a4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(sg[ks], by[ks], a4, 0, 0, 0);
      f32x4 sm;
#pragma unroll
      for (int i = 0; i < 4; ++i) sm[i] = (a4[i] + gm_xor8(a4[i])) * yunscale;
      // lane (query nl, kq) holds tokens 16 u + 4 kq .. + 3
      if (nl < NQ) *reinterpret_cast<f32x4*>(zs + nl * kGqaChunk + 16 * u + 4 * kq) = sm;
    }
    __asm__ volatile("" ::: "memory");
    float sq[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) sq[b] = zs[(2 * b + h) * kGqaChunk + r];
    __asm__ volatile("" ::: "memory");
    const bool valid = base + r < ntok;
    const float n = (float)__builtin_bit_cast(_Float16, kk.nb);
#pragma unroll
    for (int b = 0; b < NB; ++b) z[b] = valid ? lam * (c * n * sq[b]) : -INFINITY;
  };

  // online softmax of the wave step for every query, then the value sums;
  // ws[b] = softmax weight x value scale of this lane's token, query 2 b + h
  auto step = [&](const Keys& kk, const Vals& vv, int base) {
    float z[NB];
    scores(kk, base, z);
    // the step's largest value scale (both halves hold the same 32 tokens),
    // reduced across the wave only when some lane's scale has a larger
    // exponent than R (otherwise max(R, E) is R)
    int Rn = R;
    if (__ballot((int)((__builtin_bit_cast(uint32_t, kk.vs) >> 23) & 0xFF) - 127 > R) != 0) {
      const float vmax = __builtin_bit_cast(
          float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, seg_max_f32<32>(kk.vs))));
      Rn = max(R, (int)((__builtin_bit_cast(uint32_t, vmax) >> 23) & 0xFF) - 127);
    }
    const float up = __builtin_ldexpf(1.0f, R - Rn);        // 1 unless R grew
    R = Rn;
    const float f = __builtin_ldexpf(1.0f, 14 - R);
    // the step's maxima, reduced across the wave only when some score
    // exceeds its query's running maximum (otherwise they stay, and every
    // factor al is exp(0) = 1)
    bool zgrow = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) zgrow |= z[b] > (h ? Mq[2 * b + 1] : Mq[2 * b]);
    float ws[NB], al[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) al[q] = 1.0f;
    if (__ballot(zgrow) != 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        // max over the 32 tokens of each half (query 2 b + half)
        uint32_t mlo, mhi;
        halves_u32(__builtin_bit_cast(uint32_t, seg_max_f32<32>(z[b])), mlo, mhi);
        const float Mn0 = __builtin_fmaxf(Mq[2 * b], __builtin_bit_cast(float, mlo));
        const float Mn1 = __builtin_fmaxf(Mq[2 * b + 1], __builtin_bit_cast(float, mhi));
        al[2 * b] = __expf(Mq[2 * b] - Mn0);
        al[2 * b + 1] = __expf(Mq[2 * b + 1] - Mn1);
        Mq[2 * b] = Mn0;
        Mq[2 * b + 1] = Mn1;
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float pz = __expf(z[b] - (h ? Mq[2 * b + 1] : Mq[2 * b]));
      Ll[b] = Ll[b] * (h ? al[2 * b + 1] : al[2 * b]) + pz;
      ws[b] = pz * kk.vs * f;
    }
    // rescale: row 4 kq + i of every lane is query (4 kq + i) mod NQ = i mod NQ;
    // skipped when every factor is exactly 1 (no query's maximum moved and R
    // did not grow: the factors are then exp(0) and 2^0), as most steps of a
    // long range are (multiplying by 1 changes nothing)
    bool moved = up != 1.0f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) moved |= al[q] != 1.0f;
    if (moved) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float fa = al[i % NQ] * up;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j][i] *= fa;
      }
    }
    // weights -> LDS -> A fragment: row nl = (part, query), tokens 8 kq .. + 7
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int b = 0; b < NB; ++b) wst[(2 * b + h) * kGqaChunk + r] = ws[b];
    __asm__ volatile("" ::: "memory");
    const int part = nl / NQ, qa = nl % NQ;
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(wst + qa * kGqaChunk + 8 * kq);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(wst + qa * kGqaChunk + 8 * kq + 4);
    __asm__ volatile("" ::: "memory");
    f16x8 afr;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = e < 4 ? w0[e] : w1[e - 4];
      const float hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v) & 0xFFFFE000u);
      const float pv = part == 0 ? hi : (part == 1 ? v - hi : 0.0f);
      afr[e] = __builtin_amdgcn_cvt_pkrtz(pv, 0.0f)[0];
    }
    // B fragment of channel group j: codes of tokens 8 kq + e, channel
    // 8 nl + j, two tokens per register: bytes (b ^ 0x80) under the exponent
    // of 1024, minus 1152 (exact)
    uint32_t xw[8][2];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xw[e][0] = vv.vc[e][0] ^ 0x80808080u;
      xw[e][1] = vv.vc[e][1] ^ 0x80808080u;
    }
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f16x8 bfr;
      const uint32_t sel = 0x0C000C00u | (uint32_t)(j & 3) | ((uint32_t)(4 + (j & 3)) << 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t pr = __builtin_amdgcn_perm(xw[2 * i + 1][j >> 2], xw[2 * i][j >> 2], sel) | 0x64006400u;
        const h2 hv = __builtin_bit_cast(h2, pr) + bias;
        bfr[2 * i] = hv[0];
        bfr[2 * i + 1] = hv[1];
      }
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(afr, bfr, acc[j], 0, 0, 0);
    }
  };

  // y of the launch's queries first (its wait leaves the first step's loads
  // in flight); dummy query slots get a zero projection
  constexpr int TH = 64 * WAVES;
  constexpr int YK = (NQ * M + TH - 1) / TH;
  float yv[YK];
#pragma unroll
  for (int k = 0; k < YK; ++k) {
    const int idx = min((int)threadIdx.x + k * TH, NQ * M - 1);
    const int q = idx / M;
    const int qc = min(q, nq_pass - 1);
    yv[k] = yall[(g * nq_total + q_off + qc) * M + (idx % M)];
    if (q >= nq_pass) yv[k] = 0.0f;
  }
  const int first = wave * kGqaChunk;
  Keys ka, kb;
  Vals va, vb;
  __builtin_amdgcn_sched_barrier(0);
  load_keys(ka, first);
  load_vals(va, first);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int k = 0; k < YK; ++k) {
    const int idx = (int)threadIdx.x + k * TH;
    if (idx < NQ * M) y[(idx / M) * kGqaYs + idx % M] = yv[k];
  }
  build_sign_table(lds_raw, threadIdx.x, TH);
  if (threadIdx.x == 0) *next_step = WAVES;
  __syncthreads();
  // per-query power-of-two scale of y, then the B fragments, each element
  // split once by one thread and read back by every wave
  if (wave < NQ) {
    const f32x4 a = reinterpret_cast<const f32x4*>(y + wave * kGqaYs)[lane];
    uint32_t mx = max(max(abs_bits(a[0]), abs_bits(a[1])), max(abs_bits(a[2]), abs_bits(a[3])));
    mx = seg_max_u32<64>(mx);
    if (lane == 0) yscale[wave] = gm_pow2_scale(mx);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 64 * 8 * 2; idx += TH) {
    // fragment (ks, l) elements 4 e4 .. 4 e4 + 3: projections
    // 64 (l / 16) + 8 ks + 4 e4 + i of query (l mod 16) mod 8
    const int l = idx & 63, ks = (idx >> 6) & 7, e4 = idx >> 9;
    const int nc = l & 15, j = nc & 7;
    f16x4 v = {(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
    if (j < NQ) {
      const float sc = yscale[j];
      const float* src = y + j * kGqaYs + 64 * (l >> 4) + 8 * ks + 4 * e4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        _Float16 h16, l16;
        gm_split(src[i] * sc, h16, l16);
        v[i] = nc >= 8 ? l16 : h16;
      }
    }
    reinterpret_cast<f16x4*>(byf + ks * 64 + l)[e4] = v;
  }
  __syncthreads();
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) by[ks] = byf[ks * 64 + lane];
  if ((nl & 7) < NQ) yunscale = 1.0f / yscale[nl & 7];   // exact: a power of two
  // 32-token steps of the range: wave w takes step w first, then claims the
  // next free step from an LDS counter when it requests one (the next
  // step's keys are requested before the current step is scored, its values
  // after), so waves that the scheduler serves faster take more steps; the
  // partials of the waves are merged below whatever tokens each one saw
  const int nsteps = (ntok + kGqaChunk - 1) / kGqaChunk;
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(next_step, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int sa = wave, sb;
  if (sa < nsteps) {
    for (;;) {
      sb = claim();
      load_keys(kb, kGqaChunk * sb);
      step(ka, va, kGqaChunk * sa);
      load_vals(vb, kGqaChunk * sb);
      if (sb >= nsteps) break;
      sa = claim();
      load_keys(ka, kGqaChunk * sa);
      step(kb, vb, kGqaChunk * sb);
      load_vals(va, kGqaChunk * sa);
      if (sa >= nsteps) break;
    }
  }

  // hi + lo rows of each query (NQ = 4: lanes kq = 0 and 1; NQ = 2: rows
  // i and i + 2 of lanes kq = 0), unscaled by 2^(R - 14), then the waves of
  // the workgroup
  // the softmax denominators: each half's 32 lanes hold query 2 b + half
  float Lq[NQ];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    uint32_t slo, shi;
    halves_u32(__builtin_bit_cast(uint32_t, seg_sum_f32<32>(Ll[b])), slo, shi);
    Lq[2 * b] = __builtin_bit_cast(float, slo);
    Lq[2 * b + 1] = __builtin_bit_cast(float, shi);
  }
  const float unscale = __builtin_ldexpf(1.0f, R - 14);
  float ov[NQ][8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      float v;
      if constexpr (NQ == 4)
        v = acc[j][q] + swz_xor16_f32(acc[j][q]);
      else
        v = acc[j][q] + acc[j][q + 2];
      ov[q][j] = v * unscale;
    }
  __syncthreads();                           // every lookup of the workgroup is done
  float* wp = wpart + wave * NQ * (D + 2);
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (lane == 0) {
      wp[q * (D + 2)] = Mq[q];
      wp[q * (D + 2) + 1] = Lq[q];
    }
    if (kq == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) wp[q * (D + 2) + 2 + 8 * nl + j] = ov[q][j];
    }
  }
  __syncthreads();
  for (int q = 0; q < nq_pass; ++q) {
    float Mw[WAVES], Ms = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      Mw[w] = wpart[(w * NQ + q) * (D + 2)];
      Ms = __builtin_fmaxf(Ms, Mw[w]);
    }
    float sc[WAVES];
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sc[w] = (Mw[w] == -INFINITY) ? 0.0f : __expf(Mw[w] - Ms);
    float* out = partials + ((g * nq_total + q_off + q) * splits + sp) * (int64_t)(D + 2);
    if (threadIdx.x == 0) {
      float Ls = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) Ls += sc[w] * wpart[(w * NQ + q) * (D + 2) + 1];
      out[0] = Ms;
      out[1] = Ls;
    }
    for (int j = threadIdx.x; j < D; j += TH) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w)
        if (sc[w] != 0.0f) acc += sc[w] * wpart[(w * NQ + q) * (D + 2) + 2 + j];
      out[2 + j] = acc;
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped-query QJL scores on the matrix cores (m = 256, fp16 S, d <= 128,
// 2 .. 8 queries per KV head).  For a tile of 16 tokens and the head's
// queries, sum_i (2 b_ti - 1) y_i is the product of the tokens' +-1 sign
// matrix (16 x 256) and the queries' projections (256 x nq), so it runs on
// v_mfma_f32_16x16x32_f16: the A operand holds the signs as binary16 +-1
// (exact), column j < 8 of the B operand the binary16 hi part of query j's
// projection and column j + 8 its lo part, and the two columns' sums are
// added.  Each projection is scaled by a power of two (exact) so that its
// largest magnitude lies in [2^14, 2^15); hi is the scaled value with its 13
// low significand bits cleared, lo the remainder rounded toward zero, so
// hi + lo is within 2^-21 of the scaled value, relative.  Products are exact
// and the accumulation is binary32: a score is within a few 2^-21
// sum_i |y_i| of the exact estimate for the same bits and projection, far
// inside the 1e-4 ||q|| ||k|| bound.  The cost per token does not grow with
// the number of queries (the byte-table lookups of the one-query kernel
// cost 32 per token and query).
//
// Signs -> A fragments as described above; the 64 lanes read a tile's
// 512 bytes of sign words in one instruction.
//
// The projections y = S q run on the same instruction first: each wave takes
// 16 rows of S (A operand: lane (r, kq) holds channels 32 ks + 8 kq .. + 7 of
// row r) against all the queries (B operand: column j and j + 8 the hi and
// lo parts of query j after its own power-of-two scaling), so S is read once
// per workgroup whatever the number of queries.
constexpr int kGmWaves = 16;
constexpr int kGmThreads = 64 * kGmWaves;
constexpr int kGmMaxNq = 8;
constexpr int kGmTiles = 4;                                    // 16-token tiles per wave step
constexpr int kGmStep = kGmWaves * 16 * kGmTiles;              // tokens per workgroup step
// LDS: +-1 table | y [8][kGmYs] | q [8][kGmQs] | q scales [8] | y scales [8]
// (binary32) | the projection's B fragments [4][64] | the scores' B fragments
// [8][64] (16 bytes each).  The rows of y and q are padded by 8 floats so that
// the 8 queries' reads at the same offset fall in 8 different bank octets.
// The B fragments are the same in every wave: each element is computed once,
// by one thread of the workgroup, and every wave reads them back.
constexpr int kGmYs = 256 + 8, kGmQs = 128 + 8;
constexpr size_t kGmLdsBytes = kSignTableBytes + (size_t)(8 * kGmYs + 8 * kGmQs + 16) * sizeof(float) +
                               (size_t)(4 + 8) * 64 * 16 + 16;   // + the step counter
typedef _Float16 gm_f16x2 __attribute__((ext_vector_type(2)));

template <typename TQ>
__global__ __launch_bounds__(kGmThreads) __attribute__((amdgpu_waves_per_eu(4)))
void scores_qjl_mfma_kernel(const TQ* __restrict__ q, int nq, const _Float16* __restrict__ S,
                            int d, const uint32_t* __restrict__ bits,
                            const uint16_t* __restrict__ norms, int64_t T, int64_t tiles,
                            int64_t tile_tokens, float* __restrict__ scores) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  float* y = reinterpret_cast<float*>(lds_raw + kSignTableBytes);   // [8][kGmYs]
  float* qs = y + 8 * kGmYs;                                       // [8][kGmQs]
  float* qscale = qs + 8 * kGmQs;                                  // [8]
  float* yscale = qscale + 8;                                      // [8]
  f16x8* bqf = reinterpret_cast<f16x8*>(yscale + 8);               // [4][64]
  f16x8* byf = bqf + 4 * 64;                                       // [8][64]
  int* next_step = reinterpret_cast<int*>(byf + 8 * 64);           // steps handed out
  const int64_t g = blockIdx.x / tiles;
  const int64_t t0 = (blockIdx.x % tiles) * tile_tokens;
  const int ntok = (int)std::min<int64_t>(tile_tokens, T - t0);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;                     // A row / B and C column of this lane
  const int kq = lane >> 4;
  const uint32_t* bblk = bits + (g * T + t0) * 8;
  const uint16_t* nblk = norms + g * T + t0;

  // this thread's query element, then S rows 16 wave .. + 15 (the first
  // barrier waits for the query only; S is needed from the projection on).
  // Loads are unconditional: chunks and elements past d or nq read a valid
  // address and are zeroed when used.
  const int qj = threadIdx.x >> 7, qc = threadIdx.x & 127;
  const float qv = to_f32(q[(g * nq + min(qj, nq - 1)) * d + min(qc, d - 1)]);
  const int nch = d / 8;                       // 16-byte chunks of an S row
  f16x8 sa[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    sa[ks] = *reinterpret_cast<const f16x8*>(S + (int64_t)(16 * wave + n) * d +
                                             8 * min(4 * ks + kq, nch - 1));

  // a wave step: 64 tokens' sign bytes and norms
  struct Step {
    u32x2 w[kGmTiles];                         // bytes 8 kq .. 8 kq + 7 of token n of tile u
    uint16_t nb;                               // norm of token `lane` of the step
  };
  auto load_step = [&](Step& s, int base) {
#pragma unroll
    for (int u = 0; u < kGmTiles; ++u) {
      const int tok = min(base + 16 * u + n, ntok - 1);
      s.w[u] = ld_stream(reinterpret_cast<const u32x2*>(bblk + (uint32_t)tok * 8u + 2u * (uint32_t)kq));
    }
    s.nb = ld_stream(nblk + min(base + lane, ntok - 1));
  };
  // The tile's 64-token steps: wave w takes steps w and w + 16 first, then
  // claims the next free step from an LDS counter each time it requests
  // one, so waves that the scheduler serves faster score more steps (with a
  // fixed share per wave the last wave of a workgroup ended ~6 us after the
  // first).  The first two steps are requested now, behind the query
  // elements and S rows (a CU returns its vector loads in issue order);
  // requesting them after the first barrier instead delayed the set-up by
  // the issue of all the waves' token loads at once.
  const int nsteps = (ntok + 16 * kGmTiles - 1) / (16 * kGmTiles);
  auto claim = [&]() {
    int v = 0;
    if (lane == 0) v = atomicAdd(next_step, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  int a0 = wave, a1 = wave + kGmWaves, a2;
  Step s0, s1, s2;
  load_step(s0, 16 * kGmTiles * a0);
  load_step(s1, 16 * kGmTiles * a1);

  build_sign_table(lds_raw, threadIdx.x, kGmThreads);
  qs[qj * kGmQs + qc] = (qj < nq && qc < d) ? qv : 0.0f;
  if (threadIdx.x == 0) *next_step = 2 * kGmWaves;
  __syncthreads();
  // binary32 queries are scaled per query by a power of two before the
  // split; binary16 ones split exactly as they are (hi = q, lo = 0)
  if constexpr (sizeof(TQ) == 4) {
    if (wave < kGmMaxNq) {
      const f32x4 a = reinterpret_cast<const f32x4*>(qs + wave * kGmQs)[lane & 31];
      uint32_t mx = max(max(abs_bits(a[0]), abs_bits(a[1])), max(abs_bits(a[2]), abs_bits(a[3])));
      mx = seg_max_u32<64>(mx);
      if (lane == 0) qscale[wave] = gm_pow2_scale(mx);
    }
    __syncthreads();
  }

  // the projection's B fragments: fragment (ks, l) element e is channel
  // 32 ks + 8 (l / 16) + e of query (l mod 16) mod 8, its hi part for
  // l mod 16 < 8, its lo part above (two elements per thread)
  {
    const int l = threadIdx.x & 63, ks = (threadIdx.x >> 6) & 3, e2 = threadIdx.x >> 8;
    const int nl = l & 15, j = nl & 7;
    const float sc = sizeof(TQ) == 4 ? qscale[j] : 1.0f;
    const float* src = qs + j * kGmQs + 32 * ks + 8 * (l >> 4) + 2 * e2;
    _Float16 h0, l0, h1, l1;
    gm_split(src[0] * sc, h0, l0);
    gm_split(src[1] * sc, h1, l1);
    reinterpret_cast<gm_f16x2*>(bqf + ks * 64 + l)[e2] = nl >= 8 ? gm_f16x2{l0, l1} : gm_f16x2{h0, h1};
  }
  __syncthreads();

  // projections: rows 16 wave + 4 kq + i of every query
  {
    const int j = n & 7;
    const bool lo = n >= 8;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f16x8 a = 4 * ks + kq < nch ? sa[ks] : f16x8{};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bqf[ks * 64 + lane], acc, 0, 0, 0);
    }
    const float unsc = sizeof(TQ) == 4 ? 1.0f / qscale[j] : 1.0f;   // exact: a power of two
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = (acc[i] + gm_xor8(acc[i])) * unsc;
      if (!lo) y[j * kGmYs + 16 * wave + 4 * kq + i] = v;
    }
  }
  __syncthreads();
  if (wave < kGmMaxNq) {
    const f32x4 a = reinterpret_cast<const f32x4*>(y + wave * kGmYs)[lane];
    uint32_t mx = max(max(abs_bits(a[0]), abs_bits(a[1])), max(abs_bits(a[2]), abs_bits(a[3])));
    mx = seg_max_u32<64>(mx);
    if (lane == 0) yscale[wave] = gm_pow2_scale(mx);
  }
  __syncthreads();

  // B fragments of the scores: fragment (ks, l) element e is projection
  // 64 (l / 16) + 8 ks + e of query (l mod 16) mod 8, hi part for
  // l mod 16 < 8, lo part above (four elements per thread)
  {
    const int l = threadIdx.x & 63, ks = (threadIdx.x >> 6) & 7, e4 = threadIdx.x >> 9;
    const int nl = l & 15, j = nl & 7;
    const float sc = yscale[j];
    const float* src = y + j * kGmYs + 64 * (l >> 4) + 8 * ks + 4 * e4;
    f16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      _Float16 h16, l16;
      gm_split(src[i] * sc, h16, l16);
      v[i] = nl >= 8 ? l16 : h16;
    }
    reinterpret_cast<f16x4*>(byf + ks * 64 + l)[e4] = v;
  }
  __syncthreads();
  f16x8 by[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) by[ks] = byf[ks * 64 + lane];
  const float unscale = 1.0f / yscale[n & 7];  // exact: a power of two
  const float c = kSqrtHalfPi / 256.0f;
  const bool writer = n < nq;
  float* sq = scores + (g * nq + (writer ? n : 0)) * T + t0;
  // whole 16-byte runs of 4 tokens when every query row starts 16-byte aligned
  const bool vec_out = ((T | t0) & 3) == 0 && ((uintptr_t)scores & 15) == 0;
  const uint32_t tbyte = 16u * (uint32_t)n;    // byte 0 of this lane's table addresses

  auto score_step = [&](const Step& s, int base) {
    const int nstep = __builtin_bit_cast(int, (float)__builtin_bit_cast(_Float16, s.nb));
#pragma unroll
    for (int u = 0; u < kGmTiles; ++u) {
      // norms of this lane's tokens 16 u + 4 kq + i, from the lanes that
      // loaded them
      float nt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        nt[i] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((16 * u + 4 * kq + i) << 2, nstep));
      // the tile's eight sign expansions first, then its eight multiplies
      f16x8 sg[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sg[ks] = sign_fragment(s.w[u], ks, tbyte);
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(sg[ks], by[ks], acc, 0, 0, 0);
      // (the scheduler would otherwise keep one read in flight)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);   // MFMA
      // this lane's tokens: 16 u + 4 kq + i of the step
      const int tt = base + 16 * u + 4 * kq;
      f32x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = ((acc[i] + gm_xor8(acc[i])) * unscale) * (c * nt[i]);
      if (writer) {
        if (vec_out && tt + 3 < ntok) {
          *reinterpret_cast<f32x4*>(sq + tt) = out;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tt + i < ntok) sq[tt + i] = out[i];
        }
      }
    }
  };
  // three steps of sign words in flight per wave; claims only grow, so the
  // first step past the tile ends the wave's work
  for (;;) {
    a2 = claim();
    load_step(s2, 16 * kGmTiles * a2);
    if (a0 >= nsteps) break;
    score_step(s0, 16 * kGmTiles * a0);
    a0 = claim();
    load_step(s0, 16 * kGmTiles * a0);
    if (a1 >= nsteps) break;
    score_step(s1, 16 * kGmTiles * a1);
    a1 = claim();
    load_step(s1, 16 * kGmTiles * a1);
    if (a2 >= nsteps) break;
    score_step(s2, 16 * kGmTiles * a2);
  }
}

bool scores_qjl_gqa_supported(int S_f16, int m, int d, int nq) {
  return S_f16 && m == kGqaM && d >= 8 && d <= 128 && d % 8 == 0 && nq >= 2 && nq <= kGmMaxNq;
}

size_t scores_qjl_gqa_lds_bytes() { return kGmLdsBytes; }

template <typename TQ>
static hipError_t scores_qjl_gqa_typed(const TQ* q, int64_t groups, int nq, const _Float16* S,
                                       int d, const uint32_t* bits, const uint16_t* norms,
                                       int64_t T, float* scores, const DeviceInfo& dev,
                                       hipStream_t st) {
  if (T <= 0 || groups <= 0) return hipSuccess;
  const size_t lds = scores_qjl_gqa_lds_bytes();
  if (lds > dev.lds_per_block) return hipErrorInvalidConfiguration;
  hipError_t e = allow_dynamic_lds(scores_qjl_mfma_kernel<TQ>, lds);
  if (e != hipSuccess) return e;
  // about one workgroup per CU (its 64 KiB table and 16 waves fill one),
  // tiles a multiple of the workgroup step
  const int64_t splits = std::max<int64_t>(1, ((int64_t)std::max(1, dev.cus) + groups - 1) / groups);
  int64_t tile = (T + splits - 1) / splits;
  tile = (tile + kGmStep - 1) / kGmStep * kGmStep;
  const int64_t tiles = (T + tile - 1) / tile;
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 22) / tiles);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t gn = std::min(max_groups, groups - g0);
    hipLaunchKernelGGL(scores_qjl_mfma_kernel<TQ>, dim3((unsigned)(gn * tiles)), dim3(kGmThreads),
                       lds, st, q + g0 * nq * d, nq, S, d, bits + g0 * T * (kGqaM / 32),
                       norms + g0 * T, T, tiles, tile, scores + g0 * nq * T);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_scores_qjl_gqa(const void* q, int q_f16, int64_t groups, int nq,
                                 const _Float16* S, int d, const uint32_t* bits,
                                 const uint16_t* norms, int64_t T, float* scores,
                                 const DeviceInfo& dev, hipStream_t st) {
  if (q_f16)
    return scores_qjl_gqa_typed(static_cast<const _Float16*>(q), groups, nq, S, d, bits, norms, T,
                                scores, dev, st);
  return scores_qjl_gqa_typed(static_cast<const float*>(q), groups, nq, S, d, bits, norms, T, scores,
                              dev, st);
}

bool decode_gqa_supported(int m, int d, int nq) { return m == kGqaM && d == kGqaD && nq >= 2; }

// Token split of the one-pass kernel: one workgroup per CU at a time (its
// tables take 128 KiB of LDS), about two rounds of them, ranges a multiple
// of the workgroup step.
DecodeSplit decode_gqa_split(int64_t groups, int64_t T, const DeviceInfo& dev) {
  DecodeSplit s;
  const int64_t target_blocks = 2LL * std::max(1, dev.cus);
  const int64_t max_splits = std::max<int64_t>(1, (T + kGqaBlockTokens - 1) / kGqaBlockTokens);
  int64_t splits = std::min(max_splits, std::max<int64_t>(1, (target_blocks + groups - 1) / groups));
  splits = std::max<int64_t>(splits, (T + (int64_t(1) << 20) - 1) >> 20);
  int64_t tps = (T + splits - 1) / splits;
  tps = (tps + kGqaBlockTokens - 1) / kGqaBlockTokens * kGqaBlockTokens;
  s.tokens_per_split = tps;
  s.splits = (T + tps - 1) / tps;
  return s;
}

size_t decode_gqa_lds_bytes(int nb) {
  const int nq = 2 * nb;
  const int waves = gqa_waves(nb);
  // the partial sums at the end reuse the sign table's space
  static_assert((size_t)12 * 4 * (kGqaD + 2) * sizeof(float) <= kSignTableBytes, "partials fit");
  return (size_t)kSignTableBytes + ((size_t)nq * kGqaYs + 4) * sizeof(float) + 8 * 64 * 16 +
         (size_t)2 * waves * nq * kGqaChunk * sizeof(float) + 16;   // + the step counter
}

hipError_t launch_decode_gqa_pass(const float* y, int64_t groups, int nq_total, int q_off,
                                  int nq_pass, const uint32_t* kbits, const uint16_t* knorms,
                                  const int8_t* vcodes, const float* vscales, int64_t T,
                                  float lam, float* partials, const DecodeSplit& sp,
                                  hipStream_t st) {
  if (nq_pass < 1 || nq_pass > 4 || q_off + nq_pass > nq_total) return hipErrorInvalidValue;
  const int nb = nq_pass <= 2 ? 1 : 2;   // table blocks of the launch
  const size_t lds = decode_gqa_lds_bytes(nb);
  const int64_t max_groups = std::max<int64_t>(1, (int64_t(1) << 24) / sp.splits);
  for (int64_t g0 = 0; g0 < groups; g0 += max_groups) {
    const int64_t gn = std::min(max_groups, groups - g0);
    const int64_t pairs = gn * sp.splits;
    const float* yp = y + g0 * nq_total * kGqaM;
    float* pp = partials + g0 * nq_total * sp.splits * (int64_t)(kGqaD + 2);
    const uint32_t* kb = kbits + g0 * T * (kGqaM / 32);
    const uint16_t* kn = knorms + g0 * T;
    const int8_t* vc = vcodes + g0 * T * kGqaD;
    const float* vs = vscales + g0 * T;
    hipError_t e;
    if (nb == 1) {
      e = allow_dynamic_lds(decode_gqa_kernel<1>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(decode_gqa_kernel<1>, dim3((unsigned)pairs), dim3(64 * gqa_waves(1)), lds, st,
                         yp, nq_total, q_off, nq_pass, kb, kn, vc, vs, T, sp.splits,
                         sp.tokens_per_split, lam, pairs, pp);
    } else {
      e = allow_dynamic_lds(decode_gqa_kernel<2>, lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(decode_gqa_kernel<2>, dim3((unsigned)pairs), dim3(64 * gqa_waves(2)), lds, st,
                         yp, nq_total, q_off, nq_pass, kb, kn, vc, vs, T, sp.splits,
                         sp.tokens_per_split, lam, pairs, pp);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvq
