// HBM stream reference for the roofline: the practical bandwidth of a plain
// stream with a given read:write mix, measured on the device at hand.
//
// rows x 2^rd_log2 16-byte chunks are read and rows x wr16 16-byte chunks
// written (row r reads src[r << rd_log2 ..), writes dst[r * wr16 .. + wr16)),
// with every load instruction of a wave covering 1 KiB of consecutive
// bytes.  A lane that writes stores its loaded chunk xor-ed with the running
// xor of everything it has read, so no load can be dropped; lanes that do
// not write store their xor only when it equals a pattern no input here
// produces.  Used by bench.py only; no part of the compression path.
#include <hip/hip_runtime.h>

#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_rw_kernel(const u32x4* __restrict__ src,
                                                        int64_t rows, int rd_log2,
                                                        u32x4* __restrict__ dst, int wr16,
                                                        u32x4* __restrict__ sink) {
  const int64_t chunks = rows << rd_log2;
  const int64_t lmask = (int64_t(1) << rd_log2) - 1;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + c);
    acc ^= v;
    const int64_t r = c >> rd_log2;
    const int l = (int)(c & lmask);
    if (l < wr16) dst[r * wr16 + l] = v ^ acc;
  }
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) sink[threadIdx.x] = acc;
}

extern "C" int kvqprobe_stream_rw(const void* src, int64_t rows, int rd_log2, void* dst,
                                  int wr16, void* sink, int blocks, hipStream_t stream) {
  if (rows < 0 || rd_log2 < 0 || rd_log2 > 10 || wr16 < 0 || wr16 > (1 << rd_log2) ||
      blocks < 1 || !src || !sink || (wr16 > 0 && !dst))
    return 1;
  hipLaunchKernelGGL(stream_rw_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), rows, rd_log2, static_cast<u32x4*>(dst), wr16,
                     static_cast<u32x4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// The QJL sketch's memory side alone (d = 128 fp16 keys, m = 256): the
// sketch's grid of 768-thread workgroups, each wave streaming 32-row tiles
// with the next tile's loads in flight (a ring of two), writing 32 B of
// words and a 2-byte norm per row, with no arithmetic beyond an xor of what
// it read.  `layout` picks how a wave's eight 16-byte loads per tile cover
// the tile's 32 rows of 256 B:
//   0  the matrix-core operand layout: each instruction 32 rows x 32 B
//      (lane l: row l mod 32, bytes 16 (l / 32) + 32 j), cached loads;
//   1  whole lines: each instruction 4 rows x 256 B, cached loads;
//   2  whole lines, nontemporal loads.
// Rows must be a multiple of 32.  Used by bench.py only.
template <int LAYOUT>
__global__ __launch_bounds__(768) void sketch_layout_stream_kernel(
    const unsigned char* __restrict__ k, int64_t rows, u32x4* __restrict__ words,
    uint16_t* __restrict__ norms) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int64_t tiles = rows / 32;
  auto load = [&](u32x4 (&b)[8], int64_t tile) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t off = LAYOUT == 0 ? (tile * 32 + col) * 256 + 16 * h + 32 * j
                                      : (tile * 32 + 4 * j + (lane >> 4)) * 256 + 16 * (lane & 15);
      const u32x4* p = reinterpret_cast<const u32x4*>(k + off);
      b[j] = LAYOUT == 2 ? __builtin_nontemporal_load(p) : *p;
    }
  };
  const int64_t stride = (int64_t)gridDim.x * 12;
  const int64_t first = (int64_t)blockIdx.x * 12 + wave;
  if (first >= tiles) return;
  u32x4 bq[2][8];
  load(bq[0], first);
  load(bq[1], first + stride < tiles ? first + stride : tiles - 1);
  for (int64_t t0 = first;; t0 += 2 * stride) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int64_t t = t0 + r * stride;  // < tiles: checked before its loads were issued
      u32x4 x = bq[r][0];
#pragma unroll
      for (int j = 1; j < 8; ++j) x ^= bq[r][j];
      const int64_t row = t * 32 + col;
      words[row * 2 + h] = x;
      if (h == 0) norms[row] = (uint16_t)(x[0] ^ x[1] ^ x[2] ^ x[3]);
      if (t + stride >= tiles) return;
      const int64_t nx = t + 2 * stride;
      load(bq[r], nx < tiles ? nx : tiles - 1);
    }
  }
}

extern "C" int kvqprobe_sketch_layout(const void* k, int64_t rows, int layout, void* words,
                                      void* norms, int blocks, hipStream_t stream) {
  if (rows <= 0 || rows % 32 != 0 || layout < 0 || layout > 2 || blocks < 1 || !k || !words ||
      !norms)
    return 1;
  auto kern = layout == 0   ? sketch_layout_stream_kernel<0>
              : layout == 1 ? sketch_layout_stream_kernel<1>
                            : sketch_layout_stream_kernel<2>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(768), 0, stream,
                     static_cast<const unsigned char*>(k), rows, static_cast<u32x4*>(words),
                     static_cast<uint16_t*>(norms));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
