"""Pins for the decode oracle: closed forms at T = 1 and T = 2, uniform
weights, permutation invariance, overflow safety, and a per-token loop in
plain Python floats on tiny inputs."""
import math

import numpy as np

from oracle import decode as D, int8, qjl


def _cache(rng, G, T, d, m):
    S = rng.standard_normal((m, d)).astype(np.float16)
    k = rng.standard_normal((G * T, d)).astype(np.float16)
    v = rng.standard_normal((G * T, d)).astype(np.float16)
    kw, kn = qjl.qjl_sketch(k, S)
    vc, vs = int8.quantize_int8(v)
    return (S, kw.reshape(G, T, -1), kn.reshape(G, T), vc.reshape(G, T, d), vs.reshape(G, T))


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    S, kw, kn, vc, vs = _cache(rng, 3, 1, 128, 256)
    q = rng.standard_normal((3, 128)).astype(np.float16)
    out = D.decode_qjl_int8(q, S, kw, kn, vc, vs, 1 / math.sqrt(128))
    assert np.array_equal(out, vc[:, 0].astype(np.float64) * vs[:, 0, None])


def test_zero_query_gives_mean_value():
    rng = np.random.default_rng(2)
    S, kw, kn, vc, vs = _cache(rng, 2, 37, 64, 128)
    q = np.zeros((2, 64), np.float16)
    out = D.decode_qjl_int8(q, S, kw, kn, vc, vs, 0.125)
    want = (vc.astype(np.float64) * vs[..., None]).mean(axis=1)
    assert np.allclose(out, want, rtol=1e-13, atol=1e-15)


def test_two_tokens_closed_form():
    """With identical sign words, sigma_1 / sigma_0 = n_1 / n_0, so the
    softmax weight of token 1 is 1 / (1 + exp(-lam (sigma_1 - sigma_0)))."""
    rng = np.random.default_rng(3)
    d, m = 128, 256
    S = rng.standard_normal((m, d)).astype(np.float16)
    k = rng.standard_normal((1, d)).astype(np.float16)
    kw1, _ = qjl.qjl_sketch(k, S)
    kw = np.repeat(kw1[None], 2, axis=1)                           # [1, 2, W]
    kn = np.array([[1.5, 4.0]], np.float16)
    vc = rng.integers(-127, 128, (1, 2, d)).astype(np.int8)
    vs = np.array([[0.5, 0.25]], np.float32)
    q = rng.standard_normal((1, d)).astype(np.float16)
    lam = 0.0883883461356163                                       # fp32-exact
    y = q.astype(np.float64) @ S.astype(np.float64).T
    acc = float(np.sum(np.where(qjl.unpack_signs(kw1, m)[0], 1.0, -1.0) * y[0]))
    sig = [math.sqrt(math.pi / 2) / m * n * acc for n in (1.5, 4.0)]
    w1 = 1.0 / (1.0 + math.exp(-lam * (sig[1] - sig[0])))
    want = (1 - w1) * vc[0, 0] * 0.5 + w1 * vc[0, 1] * 0.25
    out = D.decode_qjl_int8(q, S, kw, kn, vc, vs, lam)
    assert np.allclose(out[0], want, rtol=1e-12, atol=1e-14)


def test_permutation_invariance():
    rng = np.random.default_rng(4)
    S, kw, kn, vc, vs = _cache(rng, 2, 50, 128, 256)
    q = rng.standard_normal((2, 128)).astype(np.float16)
    out = D.decode_qjl_int8(q, S, kw, kn, vc, vs, 1 / math.sqrt(128))
    p = rng.permutation(50)
    out2 = D.decode_qjl_int8(q, S, kw[:, p], kn[:, p], vc[:, p], vs[:, p], 1 / math.sqrt(128))
    assert np.allclose(out, out2, rtol=1e-12, atol=1e-14)


def test_large_scores_do_not_overflow():
    rng = np.random.default_rng(5)
    S, kw, kn, vc, vs = _cache(rng, 1, 64, 128, 256)
    kn = np.full_like(kn, 60000.0)
    q = (rng.standard_normal((1, 128)) * 100).astype(np.float16)
    out = D.decode_qjl_int8(q, S, kw, kn, vc, vs, 1.0)
    vh = vc.astype(np.float64) * vs[..., None]
    assert np.all(np.isfinite(out))
    assert np.all(out[0] <= vh[0].max(axis=0) + 1e-12) and np.all(out[0] >= vh[0].min(axis=0) - 1e-12)


def test_matches_per_token_python_loop():
    rng = np.random.default_rng(6)
    d, m, T = 16, 64, 9
    S, kw, kn, vc, vs = _cache(rng, 1, T, d, m)
    q = rng.standard_normal((1, d)).astype(np.float16)
    lam = 0.25
    Sf = [[float(S[i, j]) for j in range(d)] for i in range(m)]
    y = [sum(Sf[i][j] * float(q[0, j]) for j in range(d)) for i in range(m)]
    z = []
    for t in range(T):
        acc = 0.0
        for i in range(m):
            bit = (int(kw[0, t, i // 32]) >> (i % 32)) & 1
            acc += y[i] if bit else -y[i]
        z.append(float(np.float32(lam)) * math.sqrt(math.pi / 2) / m * float(kn[0, t]) * acc)
    zmax = max(z)
    e = [math.exp(v - zmax) for v in z]
    tot = sum(e)
    want = [sum(e[t] / tot * int(vc[0, t, j]) * float(vs[0, t]) for t in range(T)) for j in range(d)]
    out = D.decode_qjl_int8(q, S, kw, kn, vc, vs, lam)
    assert np.allclose(out[0], want, rtol=1e-11, atol=1e-13)
