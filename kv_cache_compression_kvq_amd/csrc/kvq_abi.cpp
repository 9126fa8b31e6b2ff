// The C ABI of libkvq: argument validation (host only, before any HIP call),
// status strings, thread-local error detail, and dispatch to the launchers.
#include "kvq.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "kvq_launch.h"

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

kvq_status ok() { return KVQ_OK; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define KVQ_CHECK_PTR(p)                                                              \
  do {                                                                                \
    if ((p) == nullptr) return fail(KVQ_ERR_NULL, "%s: %s is NULL", fn, #p);          \
    if (!aligned16(p)) return fail(KVQ_ERR_ALIGN, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

kvq_status check_dtype(const char* fn, const char* name, kvq_dtype dt) {
  if (dt != KVQ_F32 && dt != KVQ_F16)
    return fail(KVQ_ERR_DTYPE, "%s: %s = %d is not KVQ_F32 (0) or KVQ_F16 (1)", fn, name, (int)dt);
  return KVQ_OK;
}

kvq_status check_d(const char* fn, int32_t d) {
  if (d < 16 || d > kvq::kMaxD || d % 16 != 0)
    return fail(KVQ_ERR_SHAPE, "%s: d = %d must be a multiple of 16 in [16, %d]", fn, (int)d,
                kvq::kMaxD);
  return KVQ_OK;
}

kvq_status check_m(const char* fn, int32_t m) {
  if (m < kvq::kMinM || m > kvq::kMaxM || m % 32 != 0)
    return fail(KVQ_ERR_SHAPE, "%s: m = %d must be a multiple of 32 in [%d, %d]", fn, (int)m,
                kvq::kMinM, kvq::kMaxM);
  return KVQ_OK;
}

kvq_status check_nq(const char* fn, int32_t nq) {
  if (nq < 1 || nq > kvq::kMaxNq)
    return fail(KVQ_ERR_SHAPE, "%s: nq = %d must be in [1, %d]", fn, (int)nq, kvq::kMaxNq);
  return KVQ_OK;
}

kvq_status check_count(const char* fn, const char* name, int64_t v) {
  if (v < 0) return fail(KVQ_ERR_SHAPE, "%s: %s = %lld is negative", fn, name, (long long)v);
  return KVQ_OK;
}

kvq_status launched(const char* fn, hipError_t e) {
  if (e != hipSuccess)
    return fail(KVQ_ERR_LAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
  g_last_error.clear();
  return KVQ_OK;
}

kvq_status device_info(const char* fn, kvq::DeviceInfo* info) {
  hipError_t e = kvq::current_device_info(info);
  if (e != hipSuccess)
    return fail(KVQ_ERR_LAUNCH, "%s: device query failed: %s", fn, hipGetErrorString(e));
  return KVQ_OK;
}

kvq_status check_group(const char* fn, int32_t d, int32_t g) {
  if (g < 16 || g % 16 != 0 || d % g != 0)
    return fail(KVQ_ERR_SHAPE, "%s: g = %d must be a multiple of 16 that divides d = %d", fn,
                (int)g, (int)d);
  return KVQ_OK;
}

kvq_status check_channel_d(const char* fn, int32_t d) {
  if (d < 16 || d > kvq::kMaxChannelD || d % 16 != 0)
    return fail(KVQ_ERR_SHAPE, "%s: d = %d must be a multiple of 16 in [16, %d]", fn, (int)d,
                kvq::kMaxChannelD);
  return KVQ_OK;
}

kvq_status decode_impl(const char* fn, const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                       const void* S, kvq_dtype S_dt, int32_t m, const uint32_t* kbits,
                       const uint16_t* knorms, const int8_t* vcodes, const float* vscales,
                       int64_t T, int32_t d, float sm_scale, void* ws, size_t ws_bytes,
                       float* out, kvq_stream_t stream, bool static_ws = false) {
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_nq(fn, nq)) || (st = check_d(fn, d)) || (st = check_m(fn, m)) ||
      (st = check_dtype(fn, "q_dt", q_dt)) || (st = check_dtype(fn, "S_dt", S_dt)))
    return st;
  if (d > kvq::kMaxDecodeD)
    return fail(KVQ_ERR_SHAPE, "%s: d = %d exceeds %d", fn, (int)d, kvq::kMaxDecodeD);
  if (groups == 0) return ok();
  if (T == 0) return fail(KVQ_ERR_SHAPE, "%s: T = 0 (attention over no tokens)", fn);
  KVQ_CHECK_PTR(q);
  KVQ_CHECK_PTR(S);
  KVQ_CHECK_PTR(kbits);
  KVQ_CHECK_PTR(knorms);
  KVQ_CHECK_PTR(vcodes);
  KVQ_CHECK_PTR(vscales);
  KVQ_CHECK_PTR(out);
  kvq::DeviceInfo dev;
  if ((st = device_info(fn, &dev))) return st;
  const size_t need = kvq::decode_workspace_bytes(groups, nq, T, d, m, dev);
  if (static_ws) {
    if (need > kvq::kStaticScratchBytes)
      return fail(KVQ_ERR_WORKSPACE,
                  "%s: groups = %lld, T = %lld, d = %d, m = %d need %zu bytes of scratch; the "
                  "static scratch array holds %zu",
                  fn, (long long)groups, (long long)T, (int)d, (int)m, need,
                  kvq::kStaticScratchBytes);
    hipError_t e = kvq::static_scratch(&ws);
    if (e != hipSuccess)
      return fail(KVQ_ERR_LAUNCH, "%s: scratch address lookup failed: %s", fn,
                  hipGetErrorString(e));
    ws_bytes = kvq::kStaticScratchBytes;
  }
  if (ws == nullptr || ws_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu", fn, ws_bytes, ws,
                need);
  if (!aligned16(ws)) return fail(KVQ_ERR_ALIGN, "%s: ws is not 16-byte aligned", fn);
  if (kvq::decode_gqa_supported(m, d, nq) && kvq::decode_gqa_lds_bytes(2) > dev.lds_per_block)
    return fail(KVQ_ERR_SHAPE, "%s: the grouped decode needs %zu bytes of LDS, the device has %zu",
                fn, kvq::decode_gqa_lds_bytes(2), dev.lds_per_block);
  if (kvq::decode_lds_bytes(m, d) > dev.lds_per_block)
    return fail(KVQ_ERR_SHAPE, "%s: m = %d, d = %d need %zu bytes of LDS, the device has %zu", fn,
                (int)m, (int)d, kvq::decode_lds_bytes(m, d), dev.lds_per_block);
  return launched(fn, kvq::launch_decode_qjl_int8(q, q_dt == KVQ_F16, groups, nq, S,
                                                  S_dt == KVQ_F16, m, kbits, knorms, vcodes,
                                                  vscales, T, d, sm_scale, ws, out, dev,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

namespace kvq {

hipError_t current_device_info(DeviceInfo* out) {
  static std::mutex mu;
  static DeviceInfo cache[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev].device != dev) {
    DeviceInfo info;
    info.device = dev;
    e = hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    int lds = 0;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return e;
    info.lds_per_block = (size_t)lds;
    cache[dev] = info;
  }
  *out = cache[dev];
  return hipSuccess;
}

}  // namespace kvq

extern "C" {

const char* kvq_status_string(kvq_status status) {
  switch (status) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_NULL: return "KVQ_ERR_NULL";
    case KVQ_ERR_SHAPE: return "KVQ_ERR_SHAPE";
    case KVQ_ERR_ALIGN: return "KVQ_ERR_ALIGN";
    case KVQ_ERR_DTYPE: return "KVQ_ERR_DTYPE";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE";
    case KVQ_ERR_LAUNCH: return "KVQ_ERR_LAUNCH";
    default: return "KVQ_ERR_UNKNOWN";
  }
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_quantize_int8(const void* x, kvq_dtype x_dt, int64_t rows, int32_t d,
                             int8_t* codes, float* scales, kvq_stream_t stream) {
  const char* fn = "kvq_quantize_int8";
  kvq_status st;
  if ((st = check_count(fn, "rows", rows)) || (st = check_d(fn, d)) ||
      (st = check_dtype(fn, "x_dt", x_dt)))
    return st;
  if (rows == 0) return ok();
  KVQ_CHECK_PTR(x);
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(scales);
  return launched(fn, kvq::launch_quantize_int8(x, x_dt == KVQ_F16, rows, d, codes, scales,
                                                reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_dequantize_int8(const int8_t* codes, const float* scales, int64_t rows, int32_t d,
                               void* out, kvq_dtype out_dt, kvq_stream_t stream) {
  const char* fn = "kvq_dequantize_int8";
  kvq_status st;
  if ((st = check_count(fn, "rows", rows)) || (st = check_d(fn, d)) ||
      (st = check_dtype(fn, "out_dt", out_dt)))
    return st;
  if (rows == 0) return ok();
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(scales);
  KVQ_CHECK_PTR(out);
  return launched(fn, kvq::launch_dequantize_int8(codes, scales, rows, d, out, out_dt == KVQ_F16,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_scores_int8(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                           const int8_t* codes, const float* scales, int64_t T, int32_t d,
                           float* scores, kvq_stream_t stream) {
  const char* fn = "kvq_scores_int8";
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_nq(fn, nq)) || (st = check_d(fn, d)) || (st = check_dtype(fn, "q_dt", q_dt)))
    return st;
  if (groups == 0 || T == 0) return ok();
  KVQ_CHECK_PTR(q);
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(scales);
  KVQ_CHECK_PTR(scores);
  return launched(fn, kvq::launch_scores_int8(q, q_dt == KVQ_F16, groups, nq, codes, scales, T, d,
                                              scores, reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_quantize_int8_channel(const void* x, kvq_dtype x_dt, int64_t groups, int64_t T,
                                     int32_t d, int8_t* codes, float* scales,
                                     kvq_stream_t stream) {
  const char* fn = "kvq_quantize_int8_channel";
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_channel_d(fn, d)) || (st = check_dtype(fn, "x_dt", x_dt)))
    return st;
  if (groups == 0 || T == 0) return ok();
  KVQ_CHECK_PTR(x);
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(scales);
  return launched(fn, kvq::launch_quantize_int8_channel(x, x_dt == KVQ_F16, groups, T, d, codes,
                                                        scales,
                                                        reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_dequantize_int8_channel(const int8_t* codes, const float* scales, int64_t groups,
                                       int64_t T, int32_t d, void* out, kvq_dtype out_dt,
                                       kvq_stream_t stream) {
  const char* fn = "kvq_dequantize_int8_channel";
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_channel_d(fn, d)) || (st = check_dtype(fn, "out_dt", out_dt)))
    return st;
  if (groups == 0 || T == 0) return ok();
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(scales);
  KVQ_CHECK_PTR(out);
  return launched(fn, kvq::launch_dequantize_int8_channel(codes, scales, groups, T, d, out,
                                                          out_dt == KVQ_F16,
                                                          reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_scores_int8_channel(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                                   const int8_t* codes, const float* scales, int64_t T, int32_t d,
                                   float* scores, kvq_stream_t stream) {
  const char* fn = "kvq_scores_int8_channel";
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_nq(fn, nq)) || (st = check_channel_d(fn, d)) ||
      (st = check_dtype(fn, "q_dt", q_dt)))
    return st;
  if (groups == 0 || T == 0) return ok();
  KVQ_CHECK_PTR(q);
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(scales);
  KVQ_CHECK_PTR(scores);
  return launched(fn, kvq::launch_scores_int8_channel(q, q_dt == KVQ_F16, groups, nq, codes, scales,
                                                      T, d, scores,
                                                      reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_quantize_int4(const void* x, kvq_dtype x_dt, int64_t rows, int32_t d, int32_t g,
                             uint8_t* codes, float* steps, float* offsets, kvq_stream_t stream) {
  const char* fn = "kvq_quantize_int4";
  kvq_status st;
  if ((st = check_count(fn, "rows", rows)) || (st = check_d(fn, d)) ||
      (st = check_group(fn, d, g)) || (st = check_dtype(fn, "x_dt", x_dt)))
    return st;
  if (rows == 0) return ok();
  KVQ_CHECK_PTR(x);
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(steps);
  KVQ_CHECK_PTR(offsets);
  return launched(fn, kvq::launch_quantize_int4(x, x_dt == KVQ_F16, rows, d, g, codes, steps,
                                                offsets, reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_dequantize_int4(const uint8_t* codes, const float* steps, const float* offsets,
                               int64_t rows, int32_t d, int32_t g, void* out, kvq_dtype out_dt,
                               kvq_stream_t stream) {
  const char* fn = "kvq_dequantize_int4";
  kvq_status st;
  if ((st = check_count(fn, "rows", rows)) || (st = check_d(fn, d)) ||
      (st = check_group(fn, d, g)) || (st = check_dtype(fn, "out_dt", out_dt)))
    return st;
  if (rows == 0) return ok();
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(steps);
  KVQ_CHECK_PTR(offsets);
  KVQ_CHECK_PTR(out);
  return launched(fn, kvq::launch_dequantize_int4(codes, steps, offsets, rows, d, g, out,
                                                  out_dt == KVQ_F16,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_residual_sketch(const void* k, kvq_dtype k_dt, int64_t rows, int32_t d, int32_t g,
                               const void* S, kvq_dtype S_dt, int32_t m, uint8_t* codes,
                               float* steps, float* offsets, uint32_t* bits, uint16_t* norms,
                               kvq_stream_t stream) {
  const char* fn = "kvq_residual_sketch";
  kvq_status st;
  if ((st = check_count(fn, "rows", rows)) || (st = check_d(fn, d)) ||
      (st = check_group(fn, d, g)) || (st = check_m(fn, m)) ||
      (st = check_dtype(fn, "k_dt", k_dt)) || (st = check_dtype(fn, "S_dt", S_dt)))
    return st;
  if (d > kvq::kMaxDecodeD)
    return fail(KVQ_ERR_SHAPE, "%s: d = %d exceeds %d", fn, (int)d, kvq::kMaxDecodeD);
  if (rows == 0) return ok();
  KVQ_CHECK_PTR(k);
  KVQ_CHECK_PTR(S);
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(steps);
  KVQ_CHECK_PTR(offsets);
  KVQ_CHECK_PTR(bits);
  KVQ_CHECK_PTR(norms);
  kvq::DeviceInfo dev;
  if ((st = device_info(fn, &dev))) return st;
  return launched(fn, kvq::launch_residual_sketch(k, k_dt == KVQ_F16, rows, d, g, S, S_dt == KVQ_F16,
                                                  m, codes, steps, offsets, bits, norms, dev,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_scores_residual(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                               const void* S, kvq_dtype S_dt, int32_t m, int32_t g,
                               const uint8_t* codes, const float* steps, const float* offsets,
                               const uint32_t* bits, const uint16_t* norms, int64_t T, int32_t d,
                               float* scores, kvq_stream_t stream) {
  const char* fn = "kvq_scores_residual";
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_nq(fn, nq)) || (st = check_d(fn, d)) || (st = check_group(fn, d, g)) ||
      (st = check_m(fn, m)) || (st = check_dtype(fn, "q_dt", q_dt)) ||
      (st = check_dtype(fn, "S_dt", S_dt)))
    return st;
  if (d > kvq::kMaxDecodeD)
    return fail(KVQ_ERR_SHAPE, "%s: d = %d exceeds %d", fn, (int)d, kvq::kMaxDecodeD);
  if (groups == 0 || T == 0) return ok();
  KVQ_CHECK_PTR(q);
  KVQ_CHECK_PTR(S);
  KVQ_CHECK_PTR(codes);
  KVQ_CHECK_PTR(steps);
  KVQ_CHECK_PTR(offsets);
  KVQ_CHECK_PTR(bits);
  KVQ_CHECK_PTR(norms);
  KVQ_CHECK_PTR(scores);
  return launched(fn, kvq::launch_scores_residual(q, q_dt == KVQ_F16, groups, nq, S,
                                                  S_dt == KVQ_F16, m, g, codes, steps, offsets,
                                                  bits, norms, T, d, scores,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_qjl_sketch(const void* k, kvq_dtype k_dt, int64_t rows, int32_t d, const void* S,
                          int32_t m, uint32_t* bits, uint16_t* norms, kvq_stream_t stream) {
  const char* fn = "kvq_qjl_sketch";
  kvq_status st;
  if ((st = check_count(fn, "rows", rows)) || (st = check_d(fn, d)) || (st = check_m(fn, m)) ||
      (st = check_dtype(fn, "k_dt", k_dt)))
    return st;
  if (rows == 0) return ok();
  KVQ_CHECK_PTR(k);
  KVQ_CHECK_PTR(S);
  KVQ_CHECK_PTR(bits);
  KVQ_CHECK_PTR(norms);
  kvq::DeviceInfo dev;
  if ((st = device_info(fn, &dev))) return st;
  return launched(fn, kvq::launch_qjl_sketch(k, k_dt == KVQ_F16, rows, d, S, m, bits, norms, dev,
                                             reinterpret_cast<hipStream_t>(stream)));
}

kvq_status kvq_scores_qjl(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                          const void* S, kvq_dtype S_dt, int32_t m, const uint32_t* bits,
                          const uint16_t* norms, int64_t T, int32_t d, float* scores,
                          kvq_stream_t stream) {
  const char* fn = "kvq_scores_qjl";
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_nq(fn, nq)) || (st = check_d(fn, d)) || (st = check_m(fn, m)) ||
      (st = check_dtype(fn, "q_dt", q_dt)) || (st = check_dtype(fn, "S_dt", S_dt)))
    return st;
  if (groups == 0 || T == 0) return ok();
  KVQ_CHECK_PTR(q);
  KVQ_CHECK_PTR(S);
  KVQ_CHECK_PTR(bits);
  KVQ_CHECK_PTR(norms);
  KVQ_CHECK_PTR(scores);
  kvq::DeviceInfo dev;
  if ((st = device_info(fn, &dev))) return st;
  return launched(fn, kvq::launch_scores_qjl(q, q_dt == KVQ_F16, groups, nq, S, S_dt == KVQ_F16, m,
                                             bits, norms, T, d, scores, dev,
                                             reinterpret_cast<hipStream_t>(stream)));
}

size_t kvq_decode_workspace_bytes(int64_t groups, int64_t T, int32_t d, int32_t m) {
  return kvq_decode_gqa_workspace_bytes(groups, 1, T, d, m);
}

size_t kvq_decode_gqa_workspace_bytes(int64_t groups, int32_t nq, int64_t T, int32_t d,
                                      int32_t m) {
  if (groups <= 0 || nq < 1 || nq > kvq::kMaxNq || T <= 0 || d < 16 || d > kvq::kMaxDecodeD ||
      d % 16 != 0 || m < kvq::kMinM || m > kvq::kMaxM || m % 32 != 0)
    return 0;
  kvq::DeviceInfo dev;
  if (kvq::current_device_info(&dev) != hipSuccess) return 0;
  return kvq::decode_workspace_bytes(groups, nq, T, d, m, dev);
}

kvq_status kvq_decode_qjl_int8(const void* q, kvq_dtype q_dt, int64_t groups, const void* S,
                               kvq_dtype S_dt, int32_t m, const uint32_t* kbits,
                               const uint16_t* knorms, const int8_t* vcodes,
                               const float* vscales, int64_t T, int32_t d, float sm_scale,
                               void* ws, size_t ws_bytes, float* out, kvq_stream_t stream) {
  return decode_impl("kvq_decode_qjl_int8", q, q_dt, groups, 1, S, S_dt, m, kbits, knorms, vcodes,
                     vscales, T, d, sm_scale, ws, ws_bytes, out, stream);
}

kvq_status kvq_decode_qjl_int8_gqa(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                                   const void* S, kvq_dtype S_dt, int32_t m,
                                   const uint32_t* kbits, const uint16_t* knorms,
                                   const int8_t* vcodes, const float* vscales, int64_t T,
                                   int32_t d, float sm_scale, void* ws, size_t ws_bytes,
                                   float* out, kvq_stream_t stream) {
  return decode_impl("kvq_decode_qjl_int8_gqa", q, q_dt, groups, nq, S, S_dt, m, kbits, knorms,
                     vcodes, vscales, T, d, sm_scale, ws, ws_bytes, out, stream);
}

kvq_status kvq_decode_qjl_int8_noalloc(const void* q, kvq_dtype q_dt, int64_t groups,
                                       const void* S, kvq_dtype S_dt, int32_t m,
                                       const uint32_t* kbits, const uint16_t* knorms,
                                       const int8_t* vcodes, const float* vscales, int64_t T,
                                       int32_t d, float sm_scale, float* out,
                                       kvq_stream_t stream) {
  return decode_impl("kvq_decode_qjl_int8_noalloc", q, q_dt, groups, 1, S, S_dt, m, kbits, knorms,
                     vcodes, vscales, T, d, sm_scale, nullptr, 0, out, stream, true);
}

kvq_status kvq_cache_append(const void* k, const void* v, kvq_dtype kv_dt, int64_t groups,
                            int32_t d, const void* S, int32_t m, int64_t T, int64_t pos,
                            uint32_t* kbits, uint16_t* knorms, int8_t* vcodes, float* vscales,
                            kvq_stream_t stream) {
  const char* fn = "kvq_cache_append";
  kvq_status st;
  if ((st = check_count(fn, "groups", groups)) || (st = check_count(fn, "T", T)) ||
      (st = check_d(fn, d)) || (st = check_m(fn, m)) || (st = check_dtype(fn, "kv_dt", kv_dt)))
    return st;
  if (d > kvq::kMaxDecodeD)
    return fail(KVQ_ERR_SHAPE, "%s: d = %d exceeds %d", fn, (int)d, kvq::kMaxDecodeD);
  if (groups == 0) return ok();
  if (pos < 0 || pos >= T)
    return fail(KVQ_ERR_SHAPE, "%s: pos = %lld is outside [0, T = %lld)", fn, (long long)pos,
                (long long)T);
  KVQ_CHECK_PTR(k);
  KVQ_CHECK_PTR(v);
  KVQ_CHECK_PTR(S);
  KVQ_CHECK_PTR(kbits);
  KVQ_CHECK_PTR(knorms);
  KVQ_CHECK_PTR(vcodes);
  KVQ_CHECK_PTR(vscales);
  return launched(fn, kvq::launch_cache_append(k, v, kv_dt == KVQ_F16, groups, d, S, m, T, pos,
                                               kbits, knorms, vcodes, vscales,
                                               reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
