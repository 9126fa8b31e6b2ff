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
