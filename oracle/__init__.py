"""Plain fp64 CPU reference for the KV-cache compression hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import anything from this package.
The product library (``kv_cache_compression_kvq_amd``) never imports it and
shares no code, table or helper with it; both sides receive the same input
bytes from ``synth_inputs``.

Everything here is written for a reader to check against the pages by eye:
numpy in float64 (exact integer arithmetic where the method is integral),
one step per line, no blocking, fusion or reordering.

Modules
-------
int8    per-row symmetric INT8 quantize / dequantize / scale-folded score
qjl     QJL key sketch (JL projection, sign bits, key norm) and the
        asymmetric inner-product estimator
decode  one decode step over a QJL-key / INT8-value cache: scores, softmax,
        weighted sum of dequantised values
int4    asymmetric group-wise INT4 quantize / dequantize
int8_channel  per-channel (over a head's tokens) INT8 quantize / dequantize / score
residual  QJL sketch of the INT4 residual and the two-stage score

Every function is pinned by CPU tests (``tests/test_oracle_*.py``) against
exact rational arithmetic, brute force on tiny inputs, closed forms and
hand-derived fixtures; none is "parity unpinned".
"""
from . import int8, int4, int8_channel, qjl, decode, residual  # noqa: F401
