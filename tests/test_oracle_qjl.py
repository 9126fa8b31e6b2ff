"""Pins for the QJL oracle: exact signs, exact norms, bit-order fixture,
Monte-Carlo unbiasedness against the closed-form variance, a deterministic
quadrature that fixes the sqrt(pi/2) constant, and closed-form special cases.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import qjl as O
import exact as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def F(v) -> Fraction:
    return Fraction(float(v))


# --- packing ------------------------------------------------------------------

def test_bit_order_fixture():
    S = np.eye(64, dtype=np.float32)
    n = 0
    for line in open(os.path.join(GOLD, "qjl_bit_order.txt")):
        if line.startswith("#") or not line.strip():
            continue
        pat, words = [p.strip() for p in line.split("|")]
        assert len(pat) == 64
        k = np.array([[{"+": 1.0, "-": -1.0, "0": 0.0}[c] for c in pat]], np.float32)
        got, _ = O.qjl_sketch(k, S)
        want = [int(w, 16) for w in words.split()]
        assert [int(v) for v in got[0]] == want, pat
        n += 1
    assert n >= 6


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(1)
    b = rng.random((9, 96)) < 0.5
    assert np.array_equal(O.unpack_signs(O.pack_signs(b), 96), b)


# --- projection signs -----------------------------------------------------------

@pytest.mark.parametrize("d", [1, 2, 3, 4])
def test_signs_match_exact_rationals(d):
    rng = np.random.default_rng(20 + d)
    m = 64
    S = rng.standard_normal((m, d)).astype(np.float16)
    k = rng.standard_normal((50, d)).astype(np.float16)
    # a few keys with exactly cancelling projections (P = 0 -> bit 1)
    k[0] = 0
    words, _ = O.qjl_sketch(k, S)
    bits = O.unpack_signs(words, m)
    for r in range(k.shape[0]):
        for i in range(m):
            P = sum(F(S[i, j]) * F(k[r, j]) for j in range(d))
            assert bits[r, i] == (P >= 0), (r, i, P)


def test_sign_invariants():
    rng = np.random.default_rng(3)
    m, d = 256, 128
    S = rng.standard_normal((m, d)).astype(np.float16)
    k = rng.standard_normal((64, d)).astype(np.float16)
    w, n = O.qjl_sketch(k, S)
    P = O.project(k, S)
    for j in (-3, 1, 4):                                   # exact power-of-two scaling
        wj, nj = O.qjl_sketch((k.astype(np.float64) * 2.0 ** j).astype(np.float16), S)
        assert np.array_equal(wj, w)
        assert np.array_equal(nj.astype(np.float64), n.astype(np.float64) * 2.0 ** j)
    wn, nn = O.qjl_sketch(-k, S)
    b, bn = O.unpack_signs(w, m), O.unpack_signs(wn, m)
    nz = P != 0
    assert np.array_equal(bn[nz], ~b[nz])
    assert np.array_equal(nn, n)
    wz, nz0 = O.qjl_sketch(np.zeros((2, d), np.float16), S)
    assert np.all(wz == 0xFFFFFFFF) and np.all(nz0 == 0)


# --- norms --------------------------------------------------------------------

def test_norms_exact():
    rng = np.random.default_rng(4)
    for dtype, d in ((np.float16, 128), (np.float32, 8), (np.float16, 3)):
        k = (rng.standard_normal((60, d)) * 10.0 ** rng.integers(-2, 3, (60, 1))).astype(dtype)
        n = O.key_norms(k)
        for r in range(k.shape[0]):
            sq = sum(F(v) * F(v) for v in k[r])
            assert Fraction(float(n[r])) == E.rn16_sqrt(sq), r


# --- the estimator --------------------------------------------------------------

def _mc_estimates(q, k, m, n_sketch, seed):
    """Estimates of <q, k> over independent Gaussian S, through the oracle's
    own sketch + score path (words and fp16 norms)."""
    out = np.empty(n_sketch)
    for t in range(n_sketch):
        S = np.random.default_rng([seed, t]).standard_normal((m, q.size))
        words, norms = O.qjl_sketch(k[None, :], S)
        out[t] = O.scores_qjl(q[None, None, :], S, words[None], norms[None])[0, 0, 0]
    return out


@pytest.mark.parametrize("case", ["general", "equal", "orthogonal"])
def test_unbiased_monte_carlo(case):
    m, N = 256, 10_000
    # keys with binary16-exact norms so the stored norm adds no bias
    k = np.array([0.75, 1.0, 0.0, 0.0], np.float16)             # ||k|| = 1.25
    q = {"general": np.array([0.5, -1.25, 2.0, 0.375], np.float16),
         "equal": k.copy(),
         "orthogonal": np.array([1.0, -0.75, 3.0, -2.0], np.float16)}[case]
    est = _mc_estimates(q, k, m, N, seed=77)
    qk = float(sum(F(a) * F(b) for a, b in zip(q, k)))
    qq, kk = float(np.sum(q.astype(np.float64) ** 2)), 1.5625
    var = ((math.pi / 2) * qq * kk - qk * qk) / m                 # closed form
    assert abs(est.mean() - qk) <= 3.0 * math.sqrt(var / N), (est.mean(), qk)
    assert abs(est.var(ddof=1) / var - 1.0) <= 0.05, (est.var(ddof=1), var)
    if case == "equal":
        assert abs(var - (math.pi / 2 - 1) * kk * kk / m) < 1e-15
    if case == "orthogonal":
        assert qk == 0.0


def test_quadrature_pins_constant_d2():
    """Deterministic S: rows at evenly spaced angles with radius sqrt(pi/2)
    (the mean radius of a 2-D standard Gaussian).  The estimate is then a
    midpoint rule for (pi/2) ||k|| * (1/2pi) int (q.u) sign(k.u) dtheta =
    <q, k>; with the sign changes on cell edges its error is O(h^2), about
    1e-7 here.  A wrong constant, sign convention or pairing of y with the
    bits moves the result by O(1)."""
    m = 4096
    theta = 2 * np.pi * (np.arange(m) + 0.5) / m
    S = math.sqrt(math.pi / 2) * np.stack([np.cos(theta), np.sin(theta)], axis=1)
    for phi_idx in (0, 5, 777):
        phi = 2 * np.pi * phi_idx / m
        for r, q in ((1.0, np.array([0.3, -1.7])), (0.5, np.array([-2.0, 0.25]))):
            k = r * np.array([math.cos(phi), math.sin(phi)])
            y = O.project_queries(q, S)
            signs = O.project(k[None, :], S) >= 0
            est = O.estimate(y[None, :], signs, np.array([r]))[0, 0]
            assert abs(est - float(q @ k)) < 1e-6 * np.linalg.norm(q) * r, (est, q @ k)


def test_closed_form_d1():
    """d = 1: estimate = sqrt(pi/2) * q * k * mean_i |S_i| exactly."""
    rng = np.random.default_rng(8)
    m = 128
    S = rng.standard_normal((m, 1))
    for q, k in ((0.75, -1.5), (-2.0, 0.125), (1.0, 1.0)):
        words, norms = O.qjl_sketch(np.array([[k]], np.float16), S)
        est = O.scores_qjl(np.array([[[q]]], np.float16), S, words[None], norms[None])[0, 0, 0]
        want = math.sqrt(math.pi / 2) * q * k * np.mean(np.abs(S))
        assert abs(est - want) <= 1e-12 * abs(want)


def test_scores_linear_in_query_and_norm():
    rng = np.random.default_rng(9)
    m, d, G, T = 256, 128, 2, 40
    S = rng.standard_normal((m, d)).astype(np.float16)
    k = rng.standard_normal((G * T, d)).astype(np.float16)
    words, norms = O.qjl_sketch(k, S)
    words, norms = words.reshape(G, T, -1), norms.reshape(G, T)
    q1 = rng.standard_normal((G, 1, d))
    q2 = rng.standard_normal((G, 1, d))
    s1 = O.scores_qjl(q1, S, words, norms)
    s2 = O.scores_qjl(q2, S, words, norms)
    s3 = O.scores_qjl(3.0 * q1 - q2, S, words, norms)
    assert np.allclose(s3, 3.0 * s1 - s2, rtol=0, atol=1e-10)
    # zero norm -> zero score; doubling a norm doubles its score
    n2 = norms.copy()
    n2[:, 0] = 0
    n2[:, 1] = (norms[:, 1].astype(np.float64) * 2).astype(np.float16)
    s4 = O.scores_qjl(q1, S, words, n2)
    assert np.all(s4[:, :, 0] == 0)
    assert np.allclose(s4[:, :, 1], 2 * s1[:, :, 1], rtol=1e-15, atol=0)


def test_storage_fixture_qjl():
    for line in open(os.path.join(GOLD, "storage_ratios.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, d, m, val = [p.strip() for p in line.split("|")]
        d, m, val = int(d), int(m), float(val)
        if name == "qjl_bits_per_elem_fp16_norm":
            k = np.zeros((4, d), np.float16)
            words, norms = O.qjl_sketch(k, np.zeros((m, d), np.float16))
            assert 8 * (words.nbytes + norms.nbytes) / k.size == val
            assert O.storage_bits_per_element(d, m) == val
        elif name == "decode_cache_bits_per_elem":
            from oracle import int8
            assert (O.storage_bits_per_element(d, m) + int8.storage_bits_per_element(d)) / 2 == val
