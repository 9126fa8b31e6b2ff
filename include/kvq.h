/*
 * kvq.h - C ABI of libkvq, a KV-cache compressor for AMD Instinct MI355X
 * (gfx950): per-row and per-channel symmetric INT8 quantization, asymmetric
 * group-wise INT4
 * quantization, the QJL key sketch and a two-stage INT4 + residual-QJL key
 * code, with decode-time scoring and attention read straight from the
 * compressed cache.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers (HBM of the current HIP device).  The
 *   caller allocates and owns every buffer; no call allocates, frees or
 *   synchronises.  Work is enqueued on `stream` (NULL = the null stream) and
 *   is complete when that stream is; calls are therefore capturable into a
 *   HIP graph.
 * - Layouts are row-major and contiguous.  A [B, H, T, d] cache is flattened
 *   to rows = B*H*T (one row = one token of one head, d contiguous values)
 *   and groups = B*H with T rows each.
 * - Element types: KVQ_F32 = IEEE binary32, KVQ_F16 = IEEE binary16.  INT8
 *   codes are int8, INT4 codes two per uint8, scales / steps / offsets
 *   binary32, sign words uint32, norms binary16 stored as uint16 bit
 *   patterns.
 * - Validation happens on the host before any HIP call and returns a status
 *   (never aborts, never throws); kvq_last_error() then describes the
 *   failure.  rows == 0 (or groups == 0 or T == 0) is a successful no-op.
 *   Base pointers must be 16-byte aligned.  A launch failure returns
 *   KVQ_ERR_LAUNCH with the runtime's message; faults inside a kernel surface
 *   at the caller's next synchronisation, as for any HIP kernel.
 * - Inputs must be finite; results for NaN/Inf inputs are unspecified.
 * - Calls are stateless and may be made from several host threads.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t, declared without the HIP headers. */
typedef struct ihipStream_t* kvq_stream_t;

typedef int32_t kvq_status;
enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,      /* a required pointer is NULL                       */
  KVQ_ERR_SHAPE = 2,     /* a size is negative, zero where it must not be,
                            or outside the supported range                   */
  KVQ_ERR_ALIGN = 3,     /* a base pointer is not 16-byte aligned            */
  KVQ_ERR_DTYPE = 4,     /* unsupported element type (or mismatched pair)    */
  KVQ_ERR_WORKSPACE = 5, /* workspace pointer NULL or smaller than required  */
  KVQ_ERR_LAUNCH = 6     /* the HIP runtime rejected a launch / device query */
};

typedef int32_t kvq_dtype;
enum { KVQ_F32 = 0, KVQ_F16 = 1 };

/* Size of the per-device scratch array used by kvq_decode_qjl_int8_noalloc. */
#define KVQ_STATIC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * kvq_quantize_int8 - per-row symmetric INT8 quantization.
 *
 * Defined by the symmetric INT8 formula of the Q-TensorFormer model card
 * (section 6, "Adaptive KV Cache Quantization & Attention-Sink Eviction"):
 * scale = max|x| / 127; code = nearest integer of x / scale, clamped to
 * [-128, 127]; and by the INT8 KV-cache paper (arXiv 2601.04719, Abstract).
 * For each row r of x [rows, d]:
 *   a_r = max_i |x_ri|
 *   s_r = RN32(a_r / 127)                       (IEEE binary32 division)
 *   c_ri = clamp(rne(RN32(x_ri / s_r)), -128, 127)
 * with rne = round to nearest integer, ties to even.  A row whose s_r is +0
 * gets s_r = +0 and all-zero codes.  Results are bit-identical to this
 * definition (no fast-math; binary32 subnormals are honoured).
 *
 * x       [rows, d] KVQ_F32 or KVQ_F16 (x_dt)
 * codes   [rows, d] int8, written
 * scales  [rows]    binary32, written
 * d       1 <= d <= 65536, d % 16 == 0
 * Errors: NULL, ALIGN, SHAPE (rows < 0 or d outside the range), DTYPE.
 */
kvq_status kvq_quantize_int8(const void* x, kvq_dtype x_dt, int64_t rows, int32_t d,
                             int8_t* codes, float* scales, kvq_stream_t stream);

/*
 * kvq_dequantize_int8 - reconstruction of quantized rows.
 *
 * Same source as kvq_quantize_int8 (the reconstruction multiplies the code
 * back by its row scale):  out_ri = RN32(c_ri * s_r); for KVQ_F16 output,
 * out_ri = RN16(RN32(c_ri * s_r)).  Bit-exact.
 *
 * codes  [rows, d] int8;  scales [rows] binary32
 * out    [rows, d] KVQ_F32 or KVQ_F16 (out_dt), written
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_dequantize_int8(const int8_t* codes, const float* scales, int64_t rows,
                               int32_t d, void* out, kvq_dtype out_dt, kvq_stream_t stream);

/*
 * kvq_scores_int8 - decode-query scores against INT8 keys, scale folded.
 *
 * The attention-score use of INT8 keys in the INT8 KV-cache paper (arXiv
 * 2601.04719, Abstract: error of attention scores computed from quantized
 * keys).  The query is not quantized; the row scale is pulled out of the dot
 * product:
 *   scores[g, j, t] = s_{g,t} * sum_i q[g, j, i] * c[g, t, i]
 * accumulated in binary32.  Agrees with the exact value within
 * 1e-5 * s_{g,t} * sum_i |q[g, j, i] * c[g, t, i]|.
 *
 * q       [groups, nq, d] KVQ_F32 or KVQ_F16 (q_dt)
 * codes   [groups, T, d] int8;  scales [groups, T] binary32
 * scores  [groups, nq, T] binary32, written
 * 1 <= nq <= 64; d as for kvq_quantize_int8.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_scores_int8(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                           const int8_t* codes, const float* scales, int64_t T, int32_t d,
                           float* scores, kvq_stream_t stream);

/*
 * kvq_quantize_int8_channel - per-channel symmetric INT8 quantization of a
 * key cache: one scale per channel of each group, over the group's tokens.
 *
 * The symmetric INT8 formula of the Q-TensorFormer model card (section 6,
 * labelled channel-wise there) with the scale taken per channel: for group
 * g (one (batch, head)) of x [T, d] and channel c,
 *   s_gc = RN32(max_t |x_gtc| / 127)
 *   c_gtc = clamp(rne(RN32(x_gtc / s_gc)), -128, 127)
 * (IEEE binary32 divisions, ties to even; a zero scale gives codes 0).
 * Bit-identical to this definition.  The scales cover the T tokens given.
 *
 * x       [groups, T, d] KVQ_F32 or KVQ_F16 (x_dt)
 * codes   [groups, T, d] int8, written (also used as scratch by the call)
 * scales  [groups, d] binary32, written
 * 16 <= d <= 8192, d % 16 == 0.  groups == 0 or T == 0 is a no-op.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_quantize_int8_channel(const void* x, kvq_dtype x_dt, int64_t groups, int64_t T,
                                     int32_t d, int8_t* codes, float* scales,
                                     kvq_stream_t stream);

/*
 * kvq_dequantize_int8_channel - reconstruction of per-channel INT8 keys:
 * out_gtc = RN32(c_gtc * s_gc); KVQ_F16 output is RN16 of it.  Bit-exact.
 *
 * codes [groups, T, d] int8;  scales [groups, d] binary32
 * out   [groups, T, d] (out_dt), written.  d as kvq_quantize_int8_channel.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_dequantize_int8_channel(const int8_t* codes, const float* scales, int64_t groups,
                                       int64_t T, int32_t d, void* out, kvq_dtype out_dt,
                                       kvq_stream_t stream);

/*
 * kvq_scores_int8_channel - decode-query scores against per-channel INT8
 * keys: scores[g, j, t] = sum_c q[g, j, c] * s_gc * c_gtc, with the channel
 * scales folded into the query (one binary32 product per channel) and
 * binary32 accumulation.  Agrees with the exact value within
 * 1e-5 * sum_c |q_c * s_gc * c_gtc|.
 *
 * q       [groups, nq, d] (q_dt);  codes [groups, T, d];  scales [groups, d]
 * scores  [groups, nq, T] binary32, written
 * 1 <= nq <= 64; d as kvq_quantize_int8_channel.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_scores_int8_channel(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                                   const int8_t* codes, const float* scales, int64_t T, int32_t d,
                                   float* scores, kvq_stream_t stream);

/*
 * kvq_quantize_int4 - asymmetric group-wise INT4 quantization.
 *
 * Defined by the asymmetric group-wise INT4 formula of the Q-TensorFormer
 * model card (section 6, "Adaptive KV Cache Quantization & Attention-Sink
 * Eviction"): step = (max - min) / 15 and offset = min over a group; code =
 * nearest integer of (x - offset) / step, clamped to [0, 15].  A group is g
 * consecutive values of one row; row r has d / g groups.  For group (r, j):
 *   z_rj = min of the group                      (exact)
 *   s_rj = RN32(RN32(max - z_rj) / 15)           (IEEE binary32)
 *   c_ri = clamp(rne(RN32(RN32(x_ri - z_rj) / s_rj)), 0, 15)
 * with rne = round to nearest integer, ties to even.  A group whose s is +0
 * gets all-zero codes.  Codes, steps and offsets are bit-identical to this
 * definition, except that the sign of a zero offset is unspecified.  A group
 * whose max - min overflows binary32 is outside the domain (its results are
 * unspecified), as is non-finite input.
 *
 * x        [rows, d] KVQ_F32 or KVQ_F16 (x_dt)
 * codes    [rows, d / 2] uint8, written: value 2i in the low nibble of
 *          byte i, value 2i + 1 in the high nibble
 * steps    [rows, d / g] binary32, written
 * offsets  [rows, d / g] binary32, written
 * d as for kvq_quantize_int8; 16 <= g, g % 16 == 0, d % g == 0.
 * Errors: NULL, ALIGN, SHAPE (rows < 0, d or g outside the range), DTYPE.
 */
kvq_status kvq_quantize_int4(const void* x, kvq_dtype x_dt, int64_t rows, int32_t d, int32_t g,
                             uint8_t* codes, float* steps, float* offsets, kvq_stream_t stream);

/*
 * kvq_dequantize_int4 - reconstruction of INT4-quantized rows.
 *
 * Same source as kvq_quantize_int4 (code times step plus offset), rounded
 * twice, never fused: out_ri = RN32(RN32(c_ri * s_rj) + z_rj); for KVQ_F16
 * output, RN16 of that binary32 value.  Bit-exact.
 *
 * codes, steps, offsets as written by kvq_quantize_int4 for the same d, g
 * out    [rows, d] KVQ_F32 or KVQ_F16 (out_dt), written
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_dequantize_int4(const uint8_t* codes, const float* steps, const float* offsets,
                               int64_t rows, int32_t d, int32_t g, void* out, kvq_dtype out_dt,
                               kvq_stream_t stream);

/*
 * kvq_qjl_sketch - QJL sketch of key rows: sign bits of a JL projection plus
 * the key norm.
 *
 * From the QJL paper (arXiv 2406.03482, abstract: a Johnson-Lindenstrauss
 * transform followed by sign-bit quantization, no stored quantization
 * constants).  For each row k_r of k [rows, d] and S [m, d]:
 *   P_ri  = sum_j S_ij k_rj            (binary32 accumulation)
 *   bit i = [P_ri >= 0], stored in word i / 32 at bit i % 32 (LSB first)
 *   norm  = RN16(sqrt(sum_j k_rj^2))   (binary32 accumulation, correctly
 *                                        rounded sqrt, then binary16)
 * A bit may differ from the exact-arithmetic sign only where
 * |P_ri| <= 1e-4 * ||S_i|| * ||k_r||; a norm may differ from RN16 of the
 * exact norm by one binary16 ulp.  KVQ_F16 keys use fp16 matrix cores with
 * binary32 accumulation (products of binary16 values are exact).
 *
 * k      [rows, d] (k_dt);  S [m, d] with the same element type as k
 * bits   [rows, m / 32] uint32, written
 * norms  [rows] binary16 bit patterns, written
 * d as for kvq_quantize_int8; 32 <= m <= 1024, m % 32 == 0.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_qjl_sketch(const void* k, kvq_dtype k_dt, int64_t rows, int32_t d,
                          const void* S, int32_t m, uint32_t* bits, uint16_t* norms,
                          kvq_stream_t stream);

/*
 * kvq_scores_qjl - asymmetric QJL inner-product estimate of decode queries
 * against sketched keys.
 *
 * From the QJL paper (arXiv 2406.03482, abstract: the other vector gets the
 * JL transform without quantization; the combination is an unbiased
 * estimate of the inner product).  With y = S q (binary32, not quantized):
 *   scores[g, j, t] = sqrt(pi/2) / m * norm_{g,t} * sum_i (2 b_{g,t,i} - 1) * y_i
 * Given identical bits and norms, agrees with the exact value within
 * 1e-4 * ||q|| * norm_{g,t}.  With 2 .. 8 queries, m = 256, binary16 S and
 * d <= 128 the head's queries are scored together on the matrix cores (the
 * results then differ from nq single-query calls by rounding, within that
 * bound); otherwise each query's scores equal a single-query call's.
 *
 * q      [groups, nq, d] (q_dt);  S [m, d] (S_dt; KVQ_F32 or KVQ_F16)
 * bits   [groups, T, m / 32] uint32;  norms [groups, T] binary16 patterns
 * scores [groups, nq, T] binary32, written
 * 1 <= nq <= 64; d, m as for kvq_qjl_sketch.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_scores_qjl(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                          const void* S, kvq_dtype S_dt, int32_t m, const uint32_t* bits,
                          const uint16_t* norms, int64_t T, int32_t d, float* scores,
                          kvq_stream_t stream);

/*
 * kvq_residual_sketch - two-stage key compression: INT4, then the QJL sketch
 * of the INT4 residual.
 *
 * From the TurboQuant news item (after ArsTechnica: a first quantizer whose
 * residual error a 1-bit QJL layer corrects), with the asymmetric group-wise
 * INT4 formula of the Q-TensorFormer model card (section 6) as the first
 * stage and the QJL sketch (arXiv 2406.03482, abstract) as the second.  For
 * each row k_r of k [rows, d]:
 *   codes, steps, offsets  exactly as kvq_quantize_int4 (bit-identical)
 *   khat_ri = RN32(RN32(c_ri * s) + z),  r_ri = RN32(k_ri - khat_ri)
 *   bit i   = [sum_j S_ij r_rj >= 0]   (LSB-first words, as kvq_qjl_sketch)
 *   norm    = RN16(||r_r||)
 * A bit may differ from the exact sign only where |sum_j S_ij r_rj| <=
 * 1e-4 * ||S_i|| * ||r_r||; a norm may differ from RN16 of the exact norm by
 * one binary16 ulp.  A row with r = 0 gets all bits 1 and norm 0.
 *
 * k        [rows, d] (k_dt);  S [m, d] (S_dt)
 * codes    [rows, d / 2] uint8;  steps, offsets [rows, d / g] binary32
 * bits     [rows, m / 32] uint32;  norms [rows] binary16 patterns; all written
 * 16 <= d <= 1024, d % 16 == 0; g as for kvq_quantize_int4; m as for
 * kvq_qjl_sketch.
 * Errors: NULL, ALIGN, SHAPE, DTYPE, LAUNCH.
 */
kvq_status kvq_residual_sketch(const void* k, kvq_dtype k_dt, int64_t rows, int32_t d, int32_t g,
                               const void* S, kvq_dtype S_dt, int32_t m, uint8_t* codes,
                               float* steps, float* offsets, uint32_t* bits, uint16_t* norms,
                               kvq_stream_t stream);

/*
 * kvq_scores_residual - decode-query scores against two-stage (INT4 +
 * residual QJL) keys: the first stage's inner product plus the QJL estimate
 * of the residual's.
 *
 * Same sources as kvq_residual_sketch.  With y = S q (binary32):
 *   scores[g, j, t] = q . khat_{g,t} + sqrt(pi/2) / m * norm_{g,t}
 *                     * sum_i (2 b_{g,t,i} - 1) * y_i
 * where khat is the INT4 reconstruction (as kvq_dequantize_int4).  Agrees
 * with the exact value within
 *   1e-5 * sum_i |q_i| * (c_i * s + |z|) + 1e-4 * ||q|| * norm_{g,t}
 * (s, z of the group of channel i): the INT4 part may be evaluated per group
 * as s * sum q_i c_i + z * sum q_i.
 *
 * q        [groups, nq, d] (q_dt);  S [m, d] (S_dt)
 * codes    [groups, T, d / 2];  steps, offsets [groups, T, d / g]
 * bits     [groups, T, m / 32];  norms [groups, T] binary16 patterns
 * scores   [groups, nq, T] binary32, written
 * 1 <= nq <= 64; d, g, m as for kvq_residual_sketch.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_scores_residual(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                               const void* S, kvq_dtype S_dt, int32_t m, int32_t g,
                               const uint8_t* codes, const float* steps, const float* offsets,
                               const uint32_t* bits, const uint16_t* norms, int64_t T, int32_t d,
                               float* scores, kvq_stream_t stream);

/*
 * kvq_decode_workspace_bytes - size of the scratch buffer kvq_decode_qjl_int8
 * needs for `groups` groups of T tokens, head dimension d and sketch size m
 * (0 for invalid arguments).  It holds the projected queries S q (groups * m
 * binary32) and the per-token-range softmax partials.  The value depends
 * only on the arguments and on the number of compute units of the current
 * device.
 */
size_t kvq_decode_workspace_bytes(int64_t groups, int64_t T, int32_t d, int32_t m);

/*
 * kvq_decode_qjl_int8 - one decode step of attention over a compressed
 * cache: QJL-sketched keys and INT8 values, one query per group.
 *
 * Composes the QJL estimate (arXiv 2406.03482, abstract) for the keys with
 * the INT8 reconstruction (Q-TensorFormer model card, section 6) for the
 * values, consumed by scaled-dot-product attention (the attention engine of
 * the same card's architecture diagram):
 *   sigma_t = QJL estimate of <q, k_t>            (as kvq_scores_qjl)
 *   p_t     = softmax_t(sm_scale * sigma_t)       (binary32)
 *   out[g, :] = sum_t p_t * vscale_t * vcodes[t, :]
 * Tokens are split across workgroups and merged with the log-sum-exp rule,
 * so the result is independent of the split up to binary32 rounding.
 * Given identical compressed inputs, each output agrees with the exact value
 * within 1e-4 * sum_t p_t * |vscale_t * vcodes[t, j]| + 1e-6.
 *
 * q       [groups, d] (q_dt);  S [m, d] (S_dt)
 * kbits   [groups, T, m / 32] uint32;  knorms [groups, T] binary16 patterns
 * vcodes  [groups, T, d] int8;  vscales [groups, T] binary32
 * ws      device scratch of ws_bytes >= kvq_decode_workspace_bytes(groups, T, d, m)
 *         bytes; its contents on entry are
 *         ignored and on exit unspecified; concurrent calls need distinct ws.
 * out     [groups, d] binary32, written
 * T >= 1 when groups > 0; 16 <= d <= 1024, d % 16 == 0; m as for kvq_qjl_sketch.
 * Errors: NULL, ALIGN, SHAPE, DTYPE, WORKSPACE.
 */
kvq_status kvq_decode_qjl_int8(const void* q, kvq_dtype q_dt, int64_t groups, const void* S,
                               kvq_dtype S_dt, int32_t m, const uint32_t* kbits,
                               const uint16_t* knorms, const int8_t* vcodes,
                               const float* vscales, int64_t T, int32_t d, float sm_scale,
                               void* ws, size_t ws_bytes, float* out, kvq_stream_t stream);

/*
 * kvq_decode_gqa_workspace_bytes - scratch size for kvq_decode_qjl_int8_gqa
 * (0 for invalid shapes or when the device cannot be queried).
 */
size_t kvq_decode_gqa_workspace_bytes(int64_t groups, int32_t nq, int64_t T, int32_t d,
                                      int32_t m);

/*
 * kvq_decode_qjl_int8_gqa - kvq_decode_qjl_int8 for grouped-query attention:
 * nq query heads share each group's compressed keys and values (the
 * Q-TensorFormer card, section 4, shares one KV head among several query
 * heads).  Every query j of group g gets the decode of that query alone,
 * within kvq_decode_qjl_int8's tolerance (nq = 1 is that call, bit for bit).
 * For m = 256, d = 128 and nq >= 2 one workgroup per (group, token range)
 * carries up to four of the group's queries through one pass over the range
 * (byte tables of all four in LDS), so the cache is read once per four query
 * heads; other shapes run one workgroup per query and range, numbered so
 * that those sharing a range run on one XCD at about the same time.
 *
 * q    [groups, nq, d] (q_dt);  out [groups, nq, d] binary32, written
 * ws   device scratch of ws_bytes >= kvq_decode_gqa_workspace_bytes(groups,
 *      nq, T, d, m); other arguments as kvq_decode_qjl_int8.
 * 1 <= nq <= 64.
 * Errors: NULL, ALIGN, SHAPE, DTYPE, WORKSPACE.
 */
kvq_status kvq_decode_qjl_int8_gqa(const void* q, kvq_dtype q_dt, int64_t groups, int32_t nq,
                                   const void* S, kvq_dtype S_dt, int32_t m,
                                   const uint32_t* kbits, const uint16_t* knorms,
                                   const int8_t* vcodes, const float* vscales, int64_t T,
                                   int32_t d, float sm_scale, void* ws, size_t ws_bytes,
                                   float* out, kvq_stream_t stream);

/*
 * kvq_decode_qjl_int8_noalloc - kvq_decode_qjl_int8 without a caller
 * workspace and without any allocation, for callers that cannot allocate
 * device memory (code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc).
 *
 * Runs the same kernels as kvq_decode_qjl_int8 with the same token split,
 * so its output is bit-identical to that call's for the same arguments.  The
 * scratch it needs (kvq_decode_workspace_bytes(groups, T, d, m) bytes: the
 * projected queries and the softmax partials) lives in a device array of
 * KVQ_STATIC_SCRATCH_BYTES bytes inside the library, one per GPU, held from
 * the library's load until the process ends.  Its contents need no
 * initialisation: every call writes each scratch value before reading it.
 * The array's device address is looked up once per device, on the first
 * call with that device current.  The call never calls hipMalloc, hipFree
 * or any allocating routine.
 *
 * All calls on one GPU share that GPU's array: two calls whose executions
 * overlap on the device (different streams, or host threads without
 * ordering between their streams) race on it and give undefined results.
 * Calls on one stream are ordered and safe.
 *
 * Arguments as kvq_decode_qjl_int8 without ws / ws_bytes.
 * Errors: NULL, ALIGN, SHAPE, DTYPE as kvq_decode_qjl_int8; WORKSPACE when
 * the call would need more than KVQ_STATIC_SCRATCH_BYTES of scratch (at
 * d = 128, m = 256 and T <= 2^20: up to about 5000 groups fit; the need is
 * 4 * groups * (m + splits * (d + 2)) bytes for the call's token split);
 * LAUNCH when the device query, the address lookup or a launch fails.
 */
kvq_status kvq_decode_qjl_int8_noalloc(const void* q, kvq_dtype q_dt, int64_t groups,
                                       const void* S, kvq_dtype S_dt, int32_t m,
                                       const uint32_t* kbits, const uint16_t* knorms,
                                       const int8_t* vcodes, const float* vscales, int64_t T,
                                       int32_t d, float sm_scale, float* out,
                                       kvq_stream_t stream);

/*
 * kvq_cache_append - compress-on-write for one decode step: the newest key
 * and value of every group are compressed and written into token position
 * `pos` of the group's compressed cache (the cache layout of
 * kvq_decode_qjl_int8), in one launch.
 *
 * Keys follow the QJL sketch (arXiv 2406.03482, abstract) as kvq_qjl_sketch
 * does: bit i of the key's row is [ (S k)_i >= 0 ], LSB-first in 32-bit
 * words, and its norm is the binary16 rounding of ||k||.  Values follow the
 * symmetric INT8 formula (Q-TensorFormer model card, section 6) exactly as
 * kvq_quantize_int8 does: codes and scale are bit-identical to it.  Sign
 * bits equal the exact signs except where |(S k)_i| <= 1e-4 ||S_i|| ||k||;
 * norms are within one binary16 ulp.  Only row `pos` of each group is
 * written.
 *
 * k, v    [groups, d] (kv_dt);  S [m, d] (kv_dt)
 * kbits   [groups, T, m / 32] uint32;  knorms [groups, T] binary16 patterns
 * vcodes  [groups, T, d] int8;  vscales [groups, T] binary32
 * 0 <= pos < T; 16 <= d <= 1024, d % 16 == 0; m as for kvq_qjl_sketch.
 * groups == 0 is a no-op.
 * Errors: NULL, ALIGN, SHAPE, DTYPE.
 */
kvq_status kvq_cache_append(const void* k, const void* v, kvq_dtype kv_dt, int64_t groups,
                            int32_t d, const void* S, int32_t m, int64_t T, int64_t pos,
                            uint32_t* kbits, uint16_t* knorms, int8_t* vcodes, float* vscales,
                            kvq_stream_t stream);

/* Human-readable name of a status code (static storage). */
const char* kvq_status_string(kvq_status status);

/* Detail of the last non-OK status returned on the calling thread
 * (thread-local; empty string if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
