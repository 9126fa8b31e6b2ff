"""QJL on the residual of a scalar quantizer (reference, fp64 / exact).

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never
imports this module.

Source passages
---------------
* TurboQuant news item (amp.my.ua, after ArsTechnica): compression in two
  stages; the first quantizer leaves a residual error, and a second stage,
  QJL, acts as a 1-bit error-correction layer on it, which makes the
  attention-score estimate more accurate.  (The first stage there is
  PolarQuant, which is not built here.)
* QJL (arXiv 2406.03482), abstract: the 1-bit sketch (signs of a Gaussian JL
  projection) and the asymmetric estimator, as in ``oracle.qjl``.
* Q-TensorFormer model card, section 6: the asymmetric group-wise INT4
  formula, as in ``oracle.int4``.

Readings taken where the pages are open
---------------------------------------
* First stage: asymmetric group-wise INT4 with group g (the scalar quantizer
  the pages define; a 4-bit first stage, as the news item's 4-bit figures).
  k_hat = the INT4 reconstruction RN32(RN32(c * s) + z).
* Residual: r = RN32(k - k_hat), binary32 (k widened exactly).
* Second stage: the QJL sketch of r with the layer's S: bits b = [S r >= 0]
  (P computed in fp64), norm n = RN16(||r||_2).
* Score: sigma = q . k_hat + sqrt(pi/2) / m * n * sum_i (2 b_i - 1) y_i,
  y = S q; the first term exact in fp64 from the stored k_hat, the second as
  ``oracle.qjl.estimate``.  Since the QJL estimate is unbiased for q . r,
  E_S[sigma] = q . k_hat + q . r = q . k up to the rounding of r.
* Storage per key row: INT4 codes and per-group step and offset, m sign bits
  and one binary16 norm.
"""
from __future__ import annotations

import numpy as np

from . import int4, qjl


def residual(k: np.ndarray, khat: np.ndarray) -> np.ndarray:
    """r = RN32(k - k_hat) for keys k (fp32 / fp16) and k_hat (fp32)."""
    # one fp64 subtraction of binary32 values, then RN32: correctly rounded
    # (double rounding is innocuous for 53 >= 2 * 24 + 2)
    diff = k.astype(np.float64) - khat.astype(np.float64)
    return diff.astype(np.float32)


def residual_compress(k: np.ndarray, S: np.ndarray, g: int):
    """Keys k [R, d] -> (codes uint8 [R, d/2], steps f32 [R, d/g],
    offsets f32 [R, d/g], sign words uint32 [R, m/32], norms f16 [R]),
    the last two of the residual."""
    codes, steps, offsets = int4.quantize_int4(k, g)
    khat = int4.dequantize_int4(codes, steps, offsets, g)
    r = residual(k, khat)
    words, norms = qjl.qjl_sketch(r, S)
    return codes, steps, offsets, words, norms


def residual_scores(q: np.ndarray, S: np.ndarray, codes: np.ndarray, steps: np.ndarray,
                    offsets: np.ndarray, words: np.ndarray, norms: np.ndarray,
                    g: int) -> np.ndarray:
    """Scores of queries q [G, nq, d] against residual-compressed keys:
    codes [G, T, d/2], steps / offsets [G, T, d/g], words [G, T, m/32],
    norms [G, T] -> sigma [G, nq, T] float64."""
    G, T, half = codes.shape
    d = 2 * half
    khat = int4.dequantize_int4(codes.reshape(G * T, half), steps.reshape(G * T, d // g),
                                offsets.reshape(G * T, d // g), g).reshape(G, T, d)
    base = np.matmul(q.astype(np.float64), np.swapaxes(khat.astype(np.float64), 1, 2))
    return base + qjl.scores_qjl(q, S, words, norms)


def storage_bits_per_element(d: int, g: int, m: int) -> float:
    """INT4 codes, step and offset per group, m sign bits and a binary16 norm."""
    return int4.storage_bits_per_element(g) + (m + 16) / d
