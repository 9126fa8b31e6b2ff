"""Per-channel symmetric INT8 quantization of a key cache (reference, fp64 /
exact).

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this module.

Source passage
--------------
* Q-TensorFormer model card, section 6 "Adaptive KV Cache Quantization &
  Attention-Sink Eviction": the symmetric INT8 formula, which the card
  labels channel-wise: the scale is the largest magnitude divided by 127,
  each value is divided by the scale, rounded to the nearest integer,
  clamped to [-128, 127], and multiplied back by the scale.

Readings taken where the passage is open
----------------------------------------
* Axis: one scale per channel of one head, the largest magnitude taken over
  that head's T cached tokens: for a group g (one (batch, head)) of keys
  x [T, d], s_gc = RN32(max_t |x_tc| / 127).  Every other rule is the
  per-row reading of ``oracle.int8``: code = clamp(rne(RN32(x / s)), -128,
  127), a zero scale gives codes 0, dequantised value RN32(c * s), fp16
  output RN16 of it.
* The scale covers the T tokens given (a whole prefilled cache); a token
  appended later would change it, which this operation does not model.
* Score of an unquantised query: sigma_t = sum_c q_c * s_c * c_tc (the
  inner product with the dequantised key, the scale inside the sum since it
  varies with the channel).

fp64 arithmetic gives the binary32 results exactly, as in ``oracle.int8``.
"""
from __future__ import annotations

import numpy as np

from .int8 import _widen, QMAX, CLAMP_LO, CLAMP_HI


def channel_scales(x: np.ndarray) -> np.ndarray:
    """s [G, d] = RN32(max_t |x[g, t, c]| / 127) for keys x [G, T, d]."""
    xw = _widen(x)
    a = np.max(np.abs(xw), axis=1) if xw.shape[1] > 0 else np.zeros((xw.shape[0], xw.shape[2]))
    return (a / QMAX).astype(np.float32)


def quantize_int8_channel(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x [G, T, d] (fp32 / fp16) -> (codes int8 [G, T, d], scales float32 [G, d])."""
    xw = _widen(x)
    s = channel_scales(x)
    sw = s.astype(np.float64)[:, None, :]                   # [G, 1, d]
    live = np.broadcast_to(s[:, None, :] != 0, xw.shape)
    safe = np.where(sw != 0, sw, 1.0)
    t = (xw / safe).astype(np.float32)                     # RN32(x / s)
    c = np.clip(np.rint(t), CLAMP_LO, CLAMP_HI)
    codes = np.where(live, c, 0).astype(np.int8)
    return codes, s


def dequantize_int8_channel(codes: np.ndarray, scales: np.ndarray,
                            out_dtype: str = "f32") -> np.ndarray:
    """x_hat [G, T, d] = RN32(c * s_c); fp16 output is RN16 of it."""
    prod = codes.astype(np.float64) * scales.astype(np.float64)[:, None, :]   # exact
    x32 = prod.astype(np.float32)
    if out_dtype == "f32":
        return x32
    if out_dtype == "f16":
        with np.errstate(over="ignore"):
            return x32.astype(np.float16)
    raise ValueError(out_dtype)


def scores_int8_channel(q: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """q [G, nq, d], codes [G, T, d], scales [G, d] -> sigma [G, nq, T]
    float64, sigma = sum_c q_c s_c c_tc."""
    qs = _widen(q, allow_f64=True) * scales.astype(np.float64)[:, None, :]   # exact products
    return np.matmul(qs, np.swapaxes(codes.astype(np.float64), 1, 2))
