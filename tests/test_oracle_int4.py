"""Pins for the INT4 oracle: exact rationals, brute force, a hand-derived
fixture and invariants of the formula.

None of these re-types the oracle's arithmetic: steps and codes are
re-derived with exact rational arithmetic (tests/exact.py), codes with an
exhaustive nearest-integer search, and the rest from hand-derived groups and
properties the formula implies.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int4 as O
import exact as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def F(v) -> Fraction:
    return Fraction(float(v))


def brute_code(t: Fraction) -> int:
    """The integer in [0, 15] nearest to t, ties to the even integer, by
    exhaustive search over the 16 codes."""
    best, best_d = None, None
    for k in range(16):
        dist = abs(Fraction(k) - t)
        if best is None or dist < best_d or (dist == best_d and k % 2 == 0):
            best, best_d = k, dist
    return best


def exact_group(vals):
    """(step, offset, codes) of one group with exact rationals and explicit
    binary32 roundings of each operation."""
    xs = [F(v) for v in vals]
    z = min(xs)
    s = E.rn32(E.rn32(max(xs) - z) / 15)
    if s == 0:
        return s, z, [0] * len(xs)
    return s, z, [brute_code(E.rn32(E.rn32(x - z) / s)) for x in xs]


def test_worked_groups_fixture():
    rows = [ln for ln in open(os.path.join(GOLD, "int4_worked_groups.txt"))
            if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 4
    for ln in rows:
        st, z, xs, cs = [p.strip() for p in ln.split("|")]
        x = np.array([float(v) for v in xs.split()], dtype=np.float32)[None, :]
        want = np.array([int(c) for c in cs.split()])
        packed, s, zz = O.quantize_int4(x, 16)
        assert np.array_equal(O.unpack_nibbles(packed)[0], want), ln
        assert float(zz[0, 0]) == float(z)
        assert float(s[0, 0]) == (0.0 if st == "-" else float(st))


@pytest.mark.parametrize("dtype,scale", [(np.float32, 1.0), (np.float32, 1e-30), (np.float16, 1.0),
                                         (np.float32, 3e4), (np.float16, 1e-3)])
def test_against_exact_rationals(dtype, scale):
    rng = np.random.default_rng(7)
    g = 16
    x = (rng.standard_normal((6, 48)) * scale).astype(dtype)
    x[0, :16] = x[0, 0]                       # a constant group
    x[1, 16:32] = np.linspace(-2, 2, 16)      # evenly spread
    packed, s, z = O.quantize_int4(x, g)
    codes = O.unpack_nibbles(packed)
    for r in range(x.shape[0]):
        for j in range(x.shape[1] // g):
            es, ez, ec = exact_group(x[r, g * j:g * (j + 1)])
            assert Fraction(float(s[r, j])) == es
            assert Fraction(float(z[r, j])) == ez
            assert list(codes[r, g * j:g * (j + 1)]) == ec, (r, j)


def test_reconstruction_exact_rationals():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 32)).astype(np.float32)
    packed, s, z = O.quantize_int4(x, 32)
    codes = O.unpack_nibbles(packed)
    xh = O.dequantize_int4(packed, s, z, 32)
    xh16 = O.dequantize_int4(packed, s, z, 32, "f16")
    for r in range(3):
        for i in range(32):
            v = E.rn32(E.rn32(int(codes[r, i]) * F(s[r, 0])) + F(z[r, 0]))
            assert Fraction(float(xh[r, i])) == v
            assert Fraction(float(xh16[r, i])) == E.rn16(v)


def test_invariants_min_max_error():
    rng = np.random.default_rng(9)
    for g in (16, 32, 64, 128):
        x = rng.standard_normal((50, 256)).astype(np.float32) * rng.uniform(0.1, 10, (50, 1))
        x = x.astype(np.float32)
        packed, s, z = O.quantize_int4(x, g)
        codes = O.unpack_nibbles(packed).reshape(50, 256 // g, g)
        xg = x.reshape(50, 256 // g, g)
        assert codes.max() <= 15
        # the minimum maps to 0 and the maximum to 15
        assert np.all(np.take_along_axis(codes, xg.argmin(axis=2)[..., None], 2) == 0)
        assert np.all(np.take_along_axis(codes, xg.argmax(axis=2)[..., None], 2) == 15)
        # error at most half a step (plus binary32 rounding of the steps)
        xh = O.dequantize_int4(packed, s, z, g).reshape(50, 256 // g, g)
        err = np.abs(xh.astype(np.float64) - xg)
        assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 1e-5) + 1e-6 * np.abs(xg))


def test_constant_and_zero_groups():
    x = np.full((2, 32), 3.25, dtype=np.float32)
    x[1] = 0.0
    packed, s, z = O.quantize_int4(x, 32)
    assert np.all(s == 0) and np.all(packed == 0)
    assert np.array_equal(z[:, 0], np.array([3.25, 0.0], dtype=np.float32))
    assert np.array_equal(O.dequantize_int4(packed, s, z, 32), x)


def test_nibble_order_and_round_trip():
    codes = np.arange(32, dtype=np.uint8).reshape(1, 32) % 16
    packed = O.pack_nibbles(codes)
    assert packed[0, 0] == 0x10 and packed[0, 1] == 0x32 and packed[0, 7] == 0xFE
    assert np.array_equal(O.unpack_nibbles(packed), codes)


def test_rejects_bad_groups_and_inputs():
    with pytest.raises(ValueError):
        O.quantize_int4(np.zeros((1, 48), np.float32), 32)
    with pytest.raises(ValueError):
        O.quantize_int4(np.zeros((1, 48), np.float32), 8)
    with pytest.raises(ValueError):
        O.quantize_int4(np.array([[np.nan] * 16], np.float32), 16)
    with pytest.raises(ValueError):
        O.quantize_int4(np.linspace(3e38, -3e38, 16, dtype=np.float32)[None, :], 16)


def test_storage_bits():
    assert O.storage_bits_per_element(32) == 6.0
    assert O.storage_bits_per_element(128) == 4.5
