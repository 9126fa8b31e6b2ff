"""Per-row symmetric INT8 quantization (reference, fp64 / exact).

Source passages
---------------
* Q-TensorFormer model card, section 6 "Adaptive KV Cache Quantization &
  Attention-Sink Eviction", symmetric INT8 formula: the scale is the largest
  magnitude divided by 127, each value is divided by the scale, rounded to
  the nearest integer, clamped to [-128, 127], and multiplied back by the
  scale to reconstruct.
* "GPU-Accelerated INT8 Quantization for KV Cache Compression in Large
  Language Models" (arXiv 2601.04719), Abstract: symmetric INT8 compression
  of the KV cache (4x smaller than fp32) judged by reconstruction error and
  by attention-score error.

Readings taken where the passages are open
------------------------------------------
* Axis: one scale per row, a row being one token of one head (d contiguous
  values).  The model card labels its formula channel-wise; the per-token
  axis is the one this library implements.
* s = RN32(a / 127) with a = max |x|, an IEEE binary32 division.
* code = clamp(rne(RN32(x / s)), -128, 127): the quotient is first rounded
  to binary32 (IEEE division), then to the nearest integer with ties to
  even.  The rounding bracket on the page has no tie rule; half-to-even is
  the reading.
* A row whose scale is +0 (all zeros, or a max so small that a/127
  underflows) gets scale +0 and all codes 0.
* Dequantised value: RN32(c * s); an fp16 output is RN16 of that binary32
  value (two roundings, by design).
* Non-finite input is outside the domain: the reference raises.

Why fp64 gives the binary32 results exactly: a, x, s are binary32 (or
binary16 widened exactly).  One fp64 operation on them followed by a cast
to binary32 is correctly rounded, because 53 >= 2*24 + 2 (double rounding
is innocuous; Figueroa, "When is double rounding innocuous?", 1995).
Products c * s need 8 + 24 bits and are exact in fp64.
"""
from __future__ import annotations

import numpy as np

QMAX = 127.0   # divisor of the absmax scale
CLAMP_LO, CLAMP_HI = -128, 127


def _widen(x: np.ndarray, allow_f64: bool = False) -> np.ndarray:
    ok = (np.float32, np.float16, np.float64) if allow_f64 else (np.float32, np.float16)
    if x.dtype not in ok:
        raise TypeError(f"expected float32/float16 input, got {x.dtype}")
    xw = x.astype(np.float64)
    if not np.all(np.isfinite(xw)):
        raise ValueError("non-finite input is outside the quantizer's domain")
    return xw


def row_scales(x: np.ndarray) -> np.ndarray:
    """s_r = RN32(max_i |x_ri| / 127) for every row of x [R, d]."""
    xw = _widen(x)
    a = np.max(np.abs(xw), axis=1) if xw.shape[1] > 0 else np.zeros(xw.shape[0])
    return (a / QMAX).astype(np.float32)


def quantize_int8(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x [R, d] (fp32 or fp16) -> (codes int8 [R, d], scales float32 [R])."""
    xw = _widen(x)
    s = row_scales(x)
    codes = np.zeros(xw.shape, dtype=np.int8)
    live = s != 0
    # t = RN32(x / s): fp64 division of two binary32 values, then one cast
    t = (xw[live] / s[live].astype(np.float64)[:, None]).astype(np.float32)
    # nearest integer, ties to even, then the clamp of the formula
    c = np.clip(np.rint(t), CLAMP_LO, CLAMP_HI)
    codes[live] = c.astype(np.int8)
    return codes, s


def dequantize_int8(codes: np.ndarray, scales: np.ndarray,
                    out_dtype: str = "f32") -> np.ndarray:
    """x_hat = RN32(c * s) [R, d]; fp16 output is RN16(RN32(c * s))."""
    prod = codes.astype(np.float64) * scales.astype(np.float64)[:, None]  # exact
    x32 = prod.astype(np.float32)
    if out_dtype == "f32":
        return x32
    if out_dtype == "f16":
        with np.errstate(over="ignore"):      # beyond fp16 range -> +-inf (RN16)
            return x32.astype(np.float16)
    raise ValueError(out_dtype)


def scores_int8(q: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Scale-folded score of unquantised queries against INT8 keys.

    q [G, nq, d] (fp32/fp16), codes [G, T, d] int8, scales [G, T] float32
    -> sigma [G, nq, T] float64 with sigma = s_t * sum_i q_i * c_ti.

    This is the inner product of the query with the dequantised key written
    with the scale pulled out of the sum (exact algebra); the query itself
    is not quantised (reading of "scale-folded").
    """
    qw = _widen(q, allow_f64=True)
    cw = codes.astype(np.float64)
    dots = np.matmul(qw, np.swapaxes(cw, 1, 2))          # [G, nq, T]
    return dots * scales.astype(np.float64)[:, None, :]


def storage_bits_per_element(d: int, scale_bits: int = 32) -> float:
    """Bits stored per cached element: 8-bit codes plus one scale per row."""
    return 8.0 + scale_bits / d
