"""Pins for the INT8 oracle: exact rationals, brute force, fixtures, closed forms.

None of these re-types the oracle's formula: quotients and scales are
re-derived with exact rational arithmetic (tests/exact.py), codes with an
exhaustive nearest-integer search, and the rest from hand-derived rows and
invariants the formula implies.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int8 as O
import exact as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def F(v) -> Fraction:
    return Fraction(float(v))


def brute_code(t: Fraction) -> int:
    """The integer in [-128, 127] nearest to t, ties to the even integer,
    by exhaustive search over all 256 codes."""
    best, best_d = None, None
    for k in range(-128, 128):
        dist = abs(Fraction(k) - t)
        if best is None or dist < best_d or (dist == best_d and k % 2 == 0):
            best, best_d = k, dist
    return best


def exact_row(x_row):
    """Scale and codes of one row, derived with exact rationals."""
    a = max(abs(F(v)) for v in x_row)
    s = E.rn32(a / 127)
    if s == 0:
        return s, [0] * len(x_row)
    codes = [brute_code(E.rn32(F(v) / s)) for v in x_row]
    return s, codes


# --- the exact helper itself -------------------------------------------------

def test_exact_helper_known_values():
    assert E.rn32(Fraction(1, 3)) == Fraction(float(np.float32(1.0 / 3.0)))
    assert np.float32(1.0 / 3.0).view(np.uint32) == 0x3EAAAAAB
    tiny = Fraction(1, 2 ** 149)
    assert E.rn32(tiny) == tiny                       # smallest subnormal
    assert E.rn32(tiny / 2) == 0                      # tie -> even (0)
    assert E.rn32(3 * tiny / 2) == 2 * tiny           # tie -> even (2 quanta)
    assert E.rn32(Fraction(2) ** 128) == math.inf
    assert E.rn16(Fraction(65519)) == 65504
    assert E.rn16(Fraction(65520)) == math.inf        # midpoint rounds to even = overflow
    assert E.rn16(Fraction(1) + Fraction(1, 2 ** 11)) == 1      # tie to even
    assert E.rn16(Fraction(1) + Fraction(3, 2 ** 11)) == 1 + Fraction(2, 2 ** 10)


# --- scale --------------------------------------------------------------------

def test_scale_matches_exact_rational():
    rng = np.random.default_rng(11)
    mags = np.concatenate([
        rng.standard_normal(300).astype(np.float32),
        (rng.standard_normal(100) * 1e30).astype(np.float32),
        (rng.standard_normal(100) * 1e-38).astype(np.float32),   # subnormal range
        np.array([2.0 ** -149, 2.0 ** -140, 127 * 2.0 ** -149, 3.4e38], np.float32)])
    x = mags.reshape(-1, 1)
    s = O.row_scales(x)
    for v, got in zip(mags, s):
        assert Fraction(float(got)) == E.rn32(abs(F(v)) / 127), v


# --- codes --------------------------------------------------------------------

def _near_tie_rows(rng, n):
    """Rows whose non-max entries sit within a few ulps of half-integers
    after division by the row scale."""
    rows = []
    for _ in range(n):
        a = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.integers(-3, 4) + 1e-3)
        s = np.float32(np.float64(a) / 127.0)
        row = [a]
        for _ in range(3):
            k = rng.integers(-127, 127) + 0.5
            base = np.float32(np.float64(k) * np.float64(s))
            steps = rng.integers(-3, 4)
            v = base
            for _ in range(abs(steps)):
                v = np.nextafter(v, np.float32(np.inf if steps > 0 else -np.inf), dtype=np.float32)
            row.append(v if abs(v) <= a else base)
        rows.append(row)
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("d", [1, 2, 3, 4])
def test_codes_exact_and_bruteforce_tiny_rows(d):
    rng = np.random.default_rng(100 + d)
    x = (rng.standard_normal((200, d)) * 10.0 ** rng.integers(-6, 6, (200, 1))).astype(np.float32)
    if d == 4:
        x = np.concatenate([x, _near_tie_rows(rng, 200)])
    codes, s = O.quantize_int8(x)
    for r in range(x.shape[0]):
        s_ex, c_ex = exact_row(x[r])
        assert Fraction(float(s[r])) == s_ex
        assert list(codes[r]) == c_ex, (x[r], codes[r], c_ex)


def test_exhaustive_fp16_inputs():
    """Every finite fp16 value x with |x| <= A, quantized in a row with max A."""
    allf = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allf = allf[np.isfinite(allf)]
    for A in [np.float16(1.0), np.float16(3.140625), np.float16(0.0009765625)]:
        xs = allf[np.abs(allf.astype(np.float64)) <= float(A)]
        rows = np.stack([np.full(xs.shape, A), xs], axis=1)
        codes, s = O.quantize_int8(rows)
        s_ex = E.rn32(F(A) / 127)
        assert Fraction(float(s[0])) == s_ex
        # the code is decided by rne(RN32(x / s)); compute the binary32
        # quotient exactly and round it by hand
        for x, c in zip(xs, codes[:, 1]):
            t = E.rn32(F(x) / s_ex)
            assert c == E.round_half_even_int(t), (x, c)
        assert np.all(codes[:, 0] == 127)


def test_worked_rows_fixture():
    path = os.path.join(GOLD, "int8_worked_rows.txt")
    n = 0
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, xs, cs = [p.strip() for p in line.split("|")]
        x = np.array([float(v) for v in xs.split()], dtype=np.float32)[None, :]
        want = [int(v) for v in cs.split()]
        codes, s = O.quantize_int8(x)
        assert list(codes[0]) == want, line
        if k == "zero":
            assert s[0] == 0 and not np.signbit(s[0])
        else:
            assert s[0] == np.float32(2.0 ** int(k)), line
        n += 1
    assert n >= 8


# --- invariants ---------------------------------------------------------------

@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_invariants(dtype):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((257, 128)).astype(dtype)
    codes, s = O.quantize_int8(x)
    assert codes.min() >= -127 and codes.max() <= 127       # -128 unreachable
    am = np.argmax(np.abs(x.astype(np.float64)), axis=1)
    top = codes[np.arange(x.shape[0]), am]
    assert np.all(np.abs(top) == 127)
    assert np.all(np.sign(top) == np.sign(x[np.arange(x.shape[0]), am].astype(np.float64)))
    # odd symmetry
    cn, sn = O.quantize_int8(-x)
    assert np.array_equal(cn, -codes) and np.array_equal(sn, s)
    # power-of-two scaling changes the scale, not the codes
    # (fp16 only upward: halving can drop bits of its small subnormals)
    for k in ((-12, -1, 1, 9) if dtype == np.float32 else (1, 3, 7)):
        xk = (x.astype(np.float64) * 2.0 ** k).astype(dtype)
        assert np.array_equal(xk.astype(np.float64), x.astype(np.float64) * 2.0 ** k)
        ck, sk = O.quantize_int8(xk)
        assert np.array_equal(ck, codes)
        assert np.array_equal(sk.astype(np.float64), s.astype(np.float64) * 2.0 ** k)


def test_all_equal_zero_and_underflow_rows():
    x = np.array([[0.3] * 8, [-5.0] * 8, [0.0] * 8, [-0.0] * 8,
                  [2.0 ** -149] + [0.0] * 7,           # a / 127 rounds to +0
                  [2.0 ** -135, -2.0 ** -136] + [0.0] * 6],  # subnormal, non-zero scale
                 dtype=np.float32)
    codes, s = O.quantize_int8(x)
    assert np.all(codes[0] == 127) and np.all(codes[1] == -127)
    for r in (2, 3, 4):
        assert s[r] == 0 and not np.signbit(s[r]) and np.all(codes[r] == 0)
    s_ex, c_ex = exact_row(x[5])
    assert s[5] != 0 and Fraction(float(s[5])) == s_ex and list(codes[5]) == c_ex
    assert c_ex[0] == 127 and c_ex[1] == -64         # -63.5 ties to -64


def test_round_trip_bound():
    """|x - x_hat| <= s/2 + s * 2^-24 * 127.5 + 2^-24 * |c s| (derived from the
    two binary32 roundings around the exact half-unit integer rounding)."""
    rng = np.random.default_rng(3)
    for dist in ("normal", "uniform"):
        if dist == "normal":
            x = rng.standard_normal((512, 128)).astype(np.float32)
        else:
            x = rng.uniform(-1, 1, (512, 128)).astype(np.float32)
        codes, s = O.quantize_int8(x)
        xh = O.dequantize_int8(codes, s).astype(np.float64)
        s64 = s.astype(np.float64)[:, None]
        err = np.abs(x.astype(np.float64) - xh)
        bound = s64 / 2 + s64 * 2.0 ** -24 * 127.5 + 2.0 ** -24 * np.abs(xh)
        assert np.all(err <= bound)
        assert np.max(err / s64) > 0.49      # the bound is nearly attained
    # U(-1, 1): max-abs error below 1/254 + rounding (context for the page's
    # "reconstruction error below 0.004")
    assert err.max() <= 1.0 / 254 + 1e-6


def test_dequant_exact():
    rng = np.random.default_rng(5)
    codes = rng.integers(-127, 128, (64, 16)).astype(np.int8)
    s = (np.abs(rng.standard_normal(64)) * 10.0 ** rng.integers(-30, 30, 64)).astype(np.float32)
    s[0] = 0.0
    s[1] = np.float32(2.0 ** -140)
    x32 = O.dequantize_int8(codes, s, "f32")
    x16 = O.dequantize_int8(codes, s, "f16")
    for r in range(64):
        for i in range(16):
            v = E.rn32(Fraction(int(codes[r, i])) * F(s[r]))
            assert Fraction(float(x32[r, i])) == v
            v16 = E.rn16(v)
            if v16 in (math.inf, -math.inf):
                assert np.isinf(x16[r, i]) and (np.sign(x16[r, i]) == np.sign(v16))
            else:
                assert Fraction(float(x16[r, i])) == v16
    assert not np.any(np.signbit(x32[codes == 0]))          # c = 0 gives +0


def test_nonfinite_raises():
    with pytest.raises(ValueError):
        O.quantize_int8(np.array([[1.0, np.nan]], np.float32))
    with pytest.raises(ValueError):
        O.quantize_int8(np.array([[np.inf, 1.0]], np.float32))


# --- scale-folded score ---------------------------------------------------------

def test_scores_exact_fp16_queries():
    rng = np.random.default_rng(9)
    G, nq, T, d = 2, 3, 5, 16
    q = rng.standard_normal((G, nq, d)).astype(np.float16)
    codes = rng.integers(-127, 128, (G, T, d)).astype(np.int8)
    s = np.abs(rng.standard_normal((G, T))).astype(np.float32)
    sig = O.scores_int8(q, codes, s)
    for g in range(G):
        for j in range(nq):
            for t in range(T):
                exact = F(s[g, t]) * sum(F(q[g, j, i]) * int(codes[g, t, i]) for i in range(d))
                mag = F(s[g, t]) * sum(abs(F(q[g, j, i]) * int(codes[g, t, i])) for i in range(d))
                assert abs(Fraction(float(sig[g, j, t])) - exact) <= mag * Fraction(1, 10 ** 12)


def test_scores_unit_queries_and_linearity():
    rng = np.random.default_rng(10)
    G, T, d = 3, 7, 32
    x = rng.standard_normal((G * T, d)).astype(np.float32)
    codes, s = O.quantize_int8(x)
    codes, s = codes.reshape(G, T, d), s.reshape(G, T)
    eye = np.broadcast_to(np.eye(d, dtype=np.float32), (G, d, d)).copy()
    sig = O.scores_int8(eye, codes, s)                       # [G, d, T]
    want = np.swapaxes(codes.astype(np.float64) * s.astype(np.float64)[..., None], 1, 2)
    assert np.array_equal(sig, want)                         # s * c_i, exactly
    # linearity: sigma(2 q1 + q2) = 2 sigma(q1) + sigma(q2) (q in fp64 so the
    # combination itself is exact)
    q1 = rng.standard_normal((G, 1, d))
    q2 = rng.standard_normal((G, 1, d))
    s1 = O.scores_int8(q1, codes, s)
    s2 = O.scores_int8(q2, codes, s)
    s3 = O.scores_int8(2.0 * q1 + q2, codes, s)
    mag = O.scores_int8(2.0 * np.abs(q1) + np.abs(q2), np.abs(codes), s)
    assert np.all(np.abs(s3 - (2.0 * s1 + s2)) <= 1e-13 * mag)


def test_scores_equal_query_dot_dequantised_key():
    rng = np.random.default_rng(12)
    G, T, d = 2, 33, 128
    x = rng.standard_normal((G * T, d)).astype(np.float32)
    codes, s = O.quantize_int8(x)
    q = rng.standard_normal((G, 2, d)).astype(np.float32)
    sig = O.scores_int8(q, codes.reshape(G, T, d), s.reshape(G, T))
    xh = O.dequantize_int8(codes, s).astype(np.float64).reshape(G, T, d)
    ref = np.matmul(q.astype(np.float64), np.swapaxes(xh, 1, 2))
    mag = np.matmul(np.abs(q.astype(np.float64)), np.swapaxes(np.abs(xh), 1, 2))
    assert np.all(np.abs(sig - ref) <= 2.0 ** -23 * mag + 1e-300)


# --- storage ------------------------------------------------------------------

def test_storage_fixture_int8():
    for line in open(os.path.join(GOLD, "storage_ratios.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, d, m, val = [p.strip() for p in line.split("|")]
        d, m, val = int(d), int(m), float(val)
        x = np.zeros((4, d), np.float32)
        codes, s = O.quantize_int8(x)
        if name == "int8_codes_only_vs_fp32_ratio":
            assert x.nbytes / codes.nbytes == val
        elif name == "int8_bits_per_elem_fp32_scale":
            assert 8 * (codes.nbytes + s.nbytes) / x.size == val
            assert O.storage_bits_per_element(d) == val
