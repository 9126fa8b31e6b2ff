"""Pins for the residual (INT4 + QJL) oracle: exact rationals on tiny
inputs, a closed-form zero-residual case, unbiasedness over independent
sketches, and the error-correction property (the estimate's regression on
q . r has slope 1 and its mean squared error falls to about
(pi/2) d / m of the first stage's).

None of these re-types the oracle: the tiny case is rederived step by step
with exact rational arithmetic and explicit roundings (tests/exact.py),
the others check properties the definitions imply.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import int4 as O4
from oracle import residual as OR
import exact as E
from test_oracle_int4 import exact_group

KAPPA = math.sqrt(math.pi / 2)


def F(v) -> Fraction:
    return Fraction(float(v))


@pytest.mark.parametrize("kdt", [np.float32, np.float16])
def test_tiny_case_exact_rationals(kdt):
    rng = np.random.default_rng(31)
    R, d, g, m = 4, 32, 16, 32
    k = (rng.standard_normal((R, d)) * rng.uniform(0.5, 4, (R, 1))).astype(kdt)
    S = rng.standard_normal((m, d)).astype(np.float16)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    codes, steps, offsets, words, norms = OR.residual_compress(k, S, g)
    sig = OR.residual_scores(q, S, codes[None], steps[None], offsets[None], words[None],
                             norms[None], g)[0, 0]
    cu = O4.unpack_nibbles(codes)
    Sf = [[F(S[i, j]) for j in range(d)] for i in range(m)]
    qf = [F(q[0, 0, j]) for j in range(d)]
    y = [sum(Sf[i][j] * qf[j] for j in range(d)) for i in range(m)]
    for r in range(R):
        khat, res = [], []
        for j in range(d // g):
            s, z, c = exact_group(k[r, g * j:g * (j + 1)])
            assert Fraction(float(steps[r, j])) == s and Fraction(float(offsets[r, j])) == z
            assert list(cu[r, g * j:g * (j + 1)]) == c
            for i, ci in enumerate(c):
                kh = E.rn32(E.rn32(ci * s) + z)
                khat.append(kh)
                res.append(E.rn32(F(k[r, g * j + i]) - kh))
        bits = [sum(Sf[i][j] * res[j] for j in range(d)) >= 0 for i in range(m)]
        want = sum(int(b) << i for i, b in enumerate(bits))
        assert int(words[r, 0]) == want, r
        n = E.rn16_sqrt(sum(x * x for x in res))
        assert Fraction(float(norms[r])) == n
        exact_sig = float(sum(qf[j] * khat[j] for j in range(d))) + \
            KAPPA / m * float(n) * float(sum(y[i] if bits[i] else -y[i] for i in range(m)))
        assert abs(sig[r] - exact_sig) <= 1e-12 * (1 + abs(exact_sig)), (r, sig[r], exact_sig)


def test_keys_on_the_grid_have_zero_residual():
    """Keys z + c s with every code 0..15 in each group: the first stage is
    exact, so r = 0, the norm is 0, every bit is 1 (S r = +0) and the score
    is q . k exactly."""
    rng = np.random.default_rng(5)
    R, d, g, m = 6, 64, 16, 64
    k = np.empty((R, d), np.float32)
    for r in range(R):
        for j in range(d // g):
            s = 2.0 ** rng.integers(-4, 3)
            z = float(rng.integers(-20, 20)) * s
            k[r, g * j:g * (j + 1)] = z + rng.permutation(16) * s
    S = rng.standard_normal((m, d)).astype(np.float32)
    codes, steps, offsets, words, norms = OR.residual_compress(k, S, g)
    assert np.all(norms == 0) and np.all(words == 0xFFFFFFFF)
    q = rng.standard_normal((1, 3, d)).astype(np.float32)
    sig = OR.residual_scores(q, S, codes[None], steps[None], offsets[None], words[None], norms[None], g)
    assert np.array_equal(sig[0], q[0].astype(np.float64) @ k.astype(np.float64).T)


def _compress_and_score(k, q, S, g):
    codes, steps, offsets, words, norms = OR.residual_compress(k, S, g)
    return OR.residual_scores(q, S, codes[None], steps[None], offsets[None], words[None],
                              norms[None], g)[0]


def test_unbiased_over_independent_sketches():
    """E_S[sigma] = q . k: over 3000 independent S the mean estimate is within
    4 standard errors of q . k, while the first stage alone is biased by q . r
    (many standard errors away)."""
    rng = np.random.default_rng(11)
    d, g, m, N = 64, 16, 64, 3000
    k = rng.standard_normal((1, d)).astype(np.float32)
    codes, steps, offsets = O4.quantize_int4(k, g)
    khat = O4.dequantize_int4(codes, steps, offsets, g).astype(np.float64)
    r = k.astype(np.float64) - khat
    q = (10 * r / np.linalg.norm(r) + 0.1 * rng.standard_normal((1, d))).astype(np.float32)[None]
    qk = float(q[0, 0].astype(np.float64) @ k[0].astype(np.float64))
    qkhat = float(q[0, 0].astype(np.float64) @ khat[0])
    est = np.array([_compress_and_score(k, q, rng.standard_normal((m, d)), g)[0, 0]
                    for _ in range(N)])
    se = est.std() / math.sqrt(N)
    assert abs(est.mean() - qk) <= 4 * se, (est.mean(), qk, se)
    assert abs(qkhat - qk) >= 8 * se, (qkhat, qk, se)


def test_error_correction_slope_and_mse():
    """One S (m = 256), 4096 N(0,1) keys (d = 128, g = 32), 8 queries: the
    second stage's estimate of q . r regresses on q . r with slope 1 (+-5 %),
    and the mean squared error of sigma against q . k is (pi/2) d / m of the
    first stage's (0.785, accepted in [0.65, 0.92])."""
    rng = np.random.default_rng(12)
    d, g, m, T, nq = 128, 32, 256, 4096, 8
    k = rng.standard_normal((T, d)).astype(np.float32)
    S = rng.standard_normal((m, d)).astype(np.float32)
    q = rng.standard_normal((1, nq, d)).astype(np.float32)
    codes, steps, offsets, words, norms = OR.residual_compress(k, S, g)
    sig = OR.residual_scores(q, S, codes[None], steps[None], offsets[None], words[None],
                             norms[None], g)[0]
    khat = O4.dequantize_int4(codes, steps, offsets, g).astype(np.float64)
    q64 = q[0].astype(np.float64)
    qk = q64 @ k.astype(np.float64).T
    qkhat = q64 @ khat.T
    qr = qk - qkhat
    corr = sig - qkhat
    slope = float((corr * qr).sum() / (qr * qr).sum())
    assert 0.95 <= slope <= 1.05, slope
    ratio = float(((sig - qk) ** 2).mean() / (qr ** 2).mean())
    assert 0.65 <= ratio <= 0.92, ratio


def test_storage_bits():
    assert OR.storage_bits_per_element(128, 32, 256) == 6.0 + 272 / 128
