// Host-side launchers implemented in the .hip files and called by the C ABI
// after validation.  Every launcher assumes validated arguments and returns
// the HIP status of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

struct DeviceInfo {
  int device = -1;
  int cus = 0;              // compute units
  size_t lds_per_block = 0; // bytes of LDS a workgroup may use
};

// Properties of the current device, cached per device id.
hipError_t current_device_info(DeviceInfo* out);

hipError_t launch_quantize_int8(const void* x, int x_f16, int64_t rows, int d, int8_t* codes,
                                float* scales, hipStream_t s);
hipError_t launch_dequantize_int8(const int8_t* codes, const float* scales, int64_t rows, int d,
                                  void* out, int out_f16, hipStream_t s);
hipError_t launch_scores_int8(const void* q, int q_f16, int64_t groups, int nq,
                              const int8_t* codes, const float* scales, int64_t T, int d,
                              float* scores, hipStream_t s);
hipError_t launch_quantize_int8_channel(const void* x, int x_f16, int64_t groups, int64_t T, int d,
                                        int8_t* codes, float* scales, hipStream_t s);
hipError_t launch_dequantize_int8_channel(const int8_t* codes, const float* scales, int64_t groups,
                                          int64_t T, int d, void* out, int out_f16, hipStream_t s);
hipError_t launch_scores_int8_channel(const void* q, int q_f16, int64_t groups, int nq,
                                      const int8_t* codes, const float* scales, int64_t T, int d,
                                      float* scores, hipStream_t s);
hipError_t launch_quantize_int4(const void* x, int x_f16, int64_t rows, int d, int g,
                                uint8_t* codes, float* steps, float* offsets, hipStream_t s);
hipError_t launch_dequantize_int4(const uint8_t* codes, const float* steps, const float* offsets,
                                  int64_t rows, int d, int g, void* out, int out_f16,
                                  hipStream_t s);
hipError_t launch_qjl_sketch(const void* k, int k_f16, int64_t rows, int d, const void* S, int m,
                             uint32_t* bits, uint16_t* norms, const DeviceInfo& dev, hipStream_t s);
hipError_t launch_scores_qjl(const void* q, int q_f16, int64_t groups, int nq, const void* S,
                             int S_f16, int m, const uint32_t* bits, const uint16_t* norms,
                             int64_t T, int d, float* scores, const DeviceInfo& dev, hipStream_t s);

hipError_t launch_residual_sketch(const void* k, int k_f16, int64_t rows, int d, int g,
                                  const void* S, int S_f16, int m, uint8_t* codes, float* steps,
                                  float* offsets, uint32_t* bits, uint16_t* norms,
                                  const DeviceInfo& dev, hipStream_t s);

hipError_t launch_scores_residual(const void* q, int q_f16, int64_t groups, int nq, const void* S,
                                  int S_f16, int m, int g, const uint8_t* codes,
                                  const float* steps, const float* offsets, const uint32_t* bits,
                                  const uint16_t* norms, int64_t T, int d, float* scores,
                                  hipStream_t s);

// Token split of the decode kernel: tokens per split and number of splits.
struct DecodeSplit {
  int64_t splits = 1;
  int64_t tokens_per_split = 0;
};
DecodeSplit decode_split(int64_t groups, int64_t T, const DeviceInfo& dev);
size_t decode_workspace_bytes(int64_t groups, int nq, int64_t T, int d, int m,
                              const DeviceInfo& dev);
size_t decode_lds_bytes(int m, int d);
hipError_t launch_decode_qjl_int8(const void* q, int q_f16, int64_t groups, int nq, const void* S,
                                  int S_f16, int m, const uint32_t* kbits, const uint16_t* knorms,
                                  const int8_t* vcodes, const float* vscales, int64_t T, int d,
                                  float sm_scale, void* ws, float* out, const DeviceInfo& dev,
                                  hipStream_t s);

// One-pass grouped-query decode (decode_gqa_kernels.hip): m = 256, d = 128,
// nq >= 2 query heads per KV head, up to four per launch.
bool decode_gqa_supported(int m, int d, int nq);
DecodeSplit decode_gqa_split(int64_t groups, int64_t T, const DeviceInfo& dev);
size_t decode_gqa_lds_bytes(int nb);
hipError_t launch_decode_gqa_pass(const float* y, int64_t groups, int nq_total, int q_off,
                                  int nq_pass, const uint32_t* kbits, const uint16_t* knorms,
                                  const int8_t* vcodes, const float* vscales, int64_t T,
                                  float lam, float* partials, const DecodeSplit& sp,
                                  hipStream_t st);

// One-pass grouped-query QJL scores (decode_gqa_kernels.hip): m = 256, fp16
// S, d <= 128, 2 .. 4 query heads per KV head; bit-identical to scoring each
// query alone.
bool scores_qjl_gqa_supported(int S_f16, int m, int d, int nq);
size_t scores_qjl_gqa_lds_bytes();
hipError_t launch_scores_qjl_gqa(const void* q, int q_f16, int64_t groups, int nq,
                                 const _Float16* S, int d, const uint32_t* bits,
                                 const uint16_t* norms, int64_t T, float* scores,
                                 const DeviceInfo& dev, hipStream_t st);

// Device address of the allocation-free decode's scratch array on the
// current device (kStaticScratchBytes bytes, 256-byte aligned; looked up
// with hipGetSymbolAddress on the first call per device).
hipError_t static_scratch(void** out);

hipError_t launch_cache_append(const void* k, const void* v, int kv_f16, int64_t groups, int d,
                               const void* S, int m, int64_t T, int64_t pos, uint32_t* kbits,
                               uint16_t* knorms, int8_t* vcodes, float* vscales, hipStream_t s);

// Raise a kernel's dynamic-LDS limit when it needs more than the default
// 64 KiB (gfx950 workgroups may use up to 160 KiB).
template <typename Kernel>
inline hipError_t allow_dynamic_lds(Kernel kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// Limits shared by validation and kernels.
constexpr int kMaxD = 65536;
constexpr int kMinM = 32;
constexpr int kMaxM = 1024;
constexpr int kMaxNq = 64;
constexpr int kMaxDecodeD = 1024;
constexpr int kMaxChannelD = 8192;   // per-channel INT8: scales and query in LDS
constexpr size_t kStaticScratchBytes = KVQ_STATIC_SCRATCH_BYTES;

}  // namespace kvq
