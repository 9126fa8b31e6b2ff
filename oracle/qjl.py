"""QJL key sketch and asymmetric inner-product estimator (reference, fp64).

Source passage
--------------
"QJL: 1-Bit Quantized JL Transform for KV Cache Quantization with Zero
Overhead" (Zandieh, Daliri, Han; arXiv 2406.03482), abstract: a key is
compressed by a Johnson-Lindenstrauss transform followed by keeping only
the sign of each coordinate; an inner product with a query is estimated
asymmetrically, by applying the same JL transform to the query without
quantising it and combining it with the key's sign bits; the estimator is
unbiased.  No per-block scale or zero point is stored.

What is computed (readings where the abstract is open)
------------------------------------------------------
* S [m, d] has i.i.d. N(0, 1) entries; it is an input (drawn by the caller
  from a seed), shared by every key and query of a layer.
* Projection  P_ri = sum_j S_ij k_rj  (fp64; products of binary16/binary32
  values are exact in fp64).
* Sign bit  b_ri = [P_ri >= 0]  (a zero projection counts as +1).
* Packing: bit i of the row lives in 32-bit word i // 32 at bit position
  i % 32 (least significant bit first).
* Key norm  n_r = RN16(sqrt(sum_j k_rj^2)), one binary16 per row.
* Query projection  y = S q  (fp64, not quantised).
* Estimate  sigma = sqrt(pi/2) / m * n * sum_i (2 b_i - 1) y_i.

The constant: for s ~ N(0, I_d), E[<s, q> sign<s, k>] = sqrt(2/pi) <q, k> /
||k|| (split q into its part along k and the orthogonal part, which is
independent of <s, k>; E|g| = sqrt(2/pi) for g ~ N(0, 1)).  Multiplying by
sqrt(pi/2) * ||k|| makes the average over the m rows unbiased for <q, k>.
"""
from __future__ import annotations

import math

import numpy as np

SQRT_HALF_PI = math.sqrt(math.pi / 2.0)


def _widen(x: np.ndarray) -> np.ndarray:
    if x.dtype not in (np.float32, np.float16, np.float64):
        raise TypeError(f"expected a float array, got {x.dtype}")
    xw = x.astype(np.float64)
    if not np.all(np.isfinite(xw)):
        raise ValueError("non-finite input is outside the sketch's domain")
    return xw


def project(k: np.ndarray, S: np.ndarray) -> np.ndarray:
    """P [R, m] with P_ri = sum_j S_ij k_rj, for keys k [R, d], S [m, d]."""
    return _widen(k) @ _widen(S).T


def pack_signs(b: np.ndarray) -> np.ndarray:
    """bool [R, m] -> uint32 [R, m // 32]; bit i -> word i // 32, bit i % 32."""
    R, m = b.shape
    if m % 32:
        raise ValueError("m must be a multiple of 32")
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    words = (b.reshape(R, m // 32, 32).astype(np.uint64) * weights).sum(axis=2)
    return words.astype(np.uint32)


def unpack_signs(words: np.ndarray, m: int) -> np.ndarray:
    """uint32 [..., m // 32] -> bool [..., m] (inverse of pack_signs)."""
    shifts = np.arange(32, dtype=np.uint32)
    bits = (words[..., :, None] >> shifts) & np.uint32(1)
    return bits.reshape(*words.shape[:-1], m).astype(bool)


def key_norms(k: np.ndarray) -> np.ndarray:
    """n_r = RN16(||k_r||_2); float64 -> float16 is a single rounding."""
    kw = _widen(k)
    with np.errstate(over="ignore"):      # beyond binary16 range -> +inf (RN16)
        return np.sqrt(np.sum(kw * kw, axis=1)).astype(np.float16)


def qjl_sketch(k: np.ndarray, S: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Keys k [R, d] -> (sign words uint32 [R, m // 32], norms float16 [R])."""
    P = project(k, S)
    return pack_signs(P >= 0.0), key_norms(k)


def project_queries(q: np.ndarray, S: np.ndarray) -> np.ndarray:
    """y = S q for queries q [..., d] -> [..., m] (no quantisation)."""
    return _widen(q) @ _widen(S).T


def estimate(y: np.ndarray, signs: np.ndarray, norms: np.ndarray) -> np.ndarray:
    """Asymmetric estimator for projected queries and sign-sketched keys.

    y [..., nq, m] fp64, signs bool [..., T, m], norms [..., T]
    -> [..., nq, T]:  sqrt(pi/2) / m * n_t * sum_i (2 b_ti - 1) y_i.
    """
    m = y.shape[-1]
    pm = np.where(signs, 1.0, -1.0)                        # 2 b - 1
    acc = np.matmul(y, np.swapaxes(pm, -1, -2))            # [..., nq, T]
    return (SQRT_HALF_PI / m) * acc * norms.astype(np.float64)[..., None, :]


def scores_qjl(q: np.ndarray, S: np.ndarray, words: np.ndarray,
               norms: np.ndarray) -> np.ndarray:
    """Scores of queries q [G, nq, d] against sketched keys.

    words [G, T, m // 32] uint32, norms [G, T] float16 (the stored values)
    -> sigma [G, nq, T] float64.
    """
    m = S.shape[0]
    y = project_queries(q, S)                              # [G, nq, m]
    return estimate(y, unpack_signs(words, m), norms)


def storage_bits_per_element(d: int, m: int, norm_bits: int = 16) -> float:
    """Bits stored per key element: m sign bits plus one norm per row."""
    return (m + norm_bits) / d
