"""One decode step over a compressed cache (reference, fp64).

Keys are QJL sketches (sign words + fp16 norms) and values are per-row INT8
codes + fp32 scales.  For each (batch, head) group with one query:

    sigma_t = QJL estimate of <q, k_t>                     (oracle.qjl)
    z_t     = lam * sigma_t,  lam = the softmax scale (1/sqrt(d) for
              standard scaled dot-product attention; an argument here)
    p_t     = exp(z_t - max z) / sum_u exp(z_u - max z)
    v_hat_t = c_t * s_t   (the dequantised value row, exact in fp64)
    out     = sum_t p_t * v_hat_t

Source passages: the QJL abstract (arXiv 2406.03482) for the key side, the
symmetric INT8 formula of the Q-TensorFormer model card (section 6) for the
value side, and the attention engine of the same card's architecture
diagram ("Joint Hybrid Execution Engine" block, scaled-dot-product
attention) for the consumer: softmax of scaled scores times values.  The pages leave the
softmax scale open; 1/sqrt(d) is the reading.
"""
from __future__ import annotations

import numpy as np

from . import qjl


def attention(scores: np.ndarray, vcodes: np.ndarray, vscales: np.ndarray,
              sm_scale: float) -> np.ndarray:
    """softmax(lam * scores) @ v_hat for scores [G, T] -> [G, d] fp64.

    ``sm_scale`` is rounded to binary32 first, as the library receives it.
    """
    lam = np.float64(np.float32(sm_scale))
    z = lam * scores
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    v_hat = vcodes.astype(np.float64) * vscales.astype(np.float64)[..., None]
    return np.einsum("gt,gtd->gd", p, v_hat)


def decode_qjl_int8(q: np.ndarray, S: np.ndarray, kwords: np.ndarray,
                    knorms: np.ndarray, vcodes: np.ndarray, vscales: np.ndarray,
                    sm_scale: float) -> np.ndarray:
    """q [G, d]; kwords [G, T, m // 32]; knorms [G, T]; vcodes [G, T, d];
    vscales [G, T] -> out [G, d] float64."""
    sigma = qjl.scores_qjl(q[:, None, :], S, kwords, knorms)[:, 0, :]
    return attention(sigma, vcodes, vscales, sm_scale)
