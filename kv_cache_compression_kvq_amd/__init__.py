"""kv_cache_compression_kvq_amd: KV-cache compression for AMD Instinct MI355X.

Per-row and per-channel symmetric INT8 quantization, asymmetric group-wise
INT4 quantization, the QJL key sketch and a two-stage INT4 + residual-QJL key
code, with decode-time scoring and attention over the compressed cache,
implemented as hand-written gfx950 HIP kernels behind the C ABI of
``include/kvq.h`` (``libkvq.so``).
This package is the thin Python binding: torch supplies device memory and
streams; every step of the computation runs in libkvq.
"""
from ._lib import KvqError, LIB_PATH, lib  # noqa: F401
from .ops import (  # noqa: F401
    cache_append,
    decode_gqa_workspace_bytes,
    decode_qjl_int8,
    decode_qjl_int8_gqa,
    decode_workspace_bytes,
    dequantize_int4,
    dequantize_int8,
    dequantize_int8_channel,
    qjl_sketch,
    residual_sketch,
    quantize_int4,
    quantize_int8,
    quantize_int8_channel,
    scores_int8,
    scores_int8_channel,
    scores_qjl,
    scores_residual,
)
