"""Helpers shared by the GPU parity tests (test code only)."""
import math
import sys

import numpy as np
import torch

import kv_cache_compression_kvq_amd as K
from oracle import qjl as OQ

DEV = "cuda"


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def up(a: np.ndarray) -> torch.Tensor:
    """Host array -> contiguous device tensor with the same bytes."""
    if a.dtype == np.uint32:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def down(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def assert_bits_within_band(gpu_words: np.ndarray, ora_words: np.ndarray, k: np.ndarray,
                            S: np.ndarray):
    """Sign bits equal the oracle's except where |P_ri| <= 1e-4 ||S_i|| ||k_r||."""
    m = S.shape[0]
    gb = OQ.unpack_signs(gpu_words.reshape(-1, m // 32), m)
    ob = OQ.unpack_signs(ora_words.reshape(-1, m // 32), m)
    diff = gb != ob
    if not diff.any():
        return 0
    r, i = np.nonzero(diff)
    k2 = k.reshape(-1, k.shape[-1]).astype(np.float64)
    S64 = S.astype(np.float64)
    P = np.einsum("rd,rd->r", k2[r], S64[i])
    band = 1e-4 * np.linalg.norm(S64[i], axis=1) * np.linalg.norm(k2[r], axis=1)
    bad = np.abs(P) > band
    assert not bad.any(), f"{bad.sum()} sign bits differ outside the 1e-4 band (first row {r[bad][0]})"
    return int(diff.sum())


def assert_norms_within_ulp(gpu_norms: np.ndarray, ora_norms: np.ndarray):
    g = gpu_norms.reshape(-1).astype(np.float16).view(np.uint16).astype(np.int64)
    o = ora_norms.reshape(-1).astype(np.float16).view(np.uint16).astype(np.int64)
    assert np.all(np.abs(g - o) <= 1), "norm differs by more than one binary16 ulp"
    return int((g != o).sum())


def assert_int8_scores(gpu, q, codes, scales, ora):
    """|gpu - ora| <= 1e-5 * s_t * sum_i |q_i c_ti| (per score)."""
    mag = np.matmul(np.abs(q.astype(np.float64)), np.swapaxes(np.abs(codes.astype(np.float64)), 1, 2))
    mag *= scales.astype(np.float64)[:, None, :]
    err = np.abs(gpu.astype(np.float64) - ora)
    assert np.all(err <= 1e-5 * mag + 1e-30), f"max rel err {np.max(err / (mag + 1e-30)):.3g}"
    return float(np.max(err / (mag + 1e-30)))


def assert_qjl_scores(gpu, q, norms, ora):
    """|gpu - ora| <= 1e-4 * ||q|| * n_t (given identical bits and norms)."""
    qn = np.linalg.norm(q.astype(np.float64), axis=-1)            # [G, nq]
    n = norms.astype(np.float64)                                  # [G, T]
    tol = 1e-4 * qn[:, :, None] * n[:, None, :]
    err = np.abs(gpu.astype(np.float64) - ora)
    assert np.all(err <= tol + 1e-30), f"max err/tol {np.max(err / (tol + 1e-30)):.3g}"
    return float(np.max(err / (tol + 1e-30)))


def decode_tolerance_check(gpu_out, q, S, kwords, knorms, vcodes, vscales, lam, ora_out):
    """|o_j - o_j^ora| <= 1e-4 * sum_t p_t |v_hat_tj| + 1e-6."""
    sig = OQ.scores_qjl(q[:, None, :], S, kwords, knorms)[:, 0, :]
    z = np.float64(np.float32(lam)) * sig
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    mag = np.einsum("gt,gtd->gd", p, np.abs(vcodes.astype(np.float64)) * vscales.astype(np.float64)[..., None])
    err = np.abs(gpu_out.astype(np.float64) - ora_out)
    tol = 1e-4 * mag + 1e-6
    assert np.all(err <= tol), f"max err/tol {np.max(err / tol):.3g}"
    return float(np.max(err / tol))
