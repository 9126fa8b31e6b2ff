"""Pins for the per-channel INT8 oracle: a hand-derived worked group, the
transpose identity with the per-row quantizer (itself pinned by exact
rationals), an exact-rational rederivation, and the score as the exact
inner product with the per-channel scaled codes."""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import int8 as O8
from oracle import int8_channel as OC
import exact as E

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _fixture():
    rec = {}
    for ln in open(os.path.join(GOLD, "int8_channel_worked.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        key, *rows = [p.strip() for p in ln.split("|")]
        rec[key] = [[float(v) for v in r.split()] for r in rows]
    return rec


def test_worked_group_fixture():
    f = _fixture()
    x = np.array(f["x"], np.float32)[None]
    codes, s = OC.quantize_int8_channel(x)
    assert np.array_equal(s[0], np.array(f["s"][0], np.float32))
    assert np.array_equal(codes[0], np.array(f["c"], np.int8))
    q = np.array(f["q"], np.float32)[None]
    assert np.array_equal(OC.scores_int8_channel(q, codes, s)[0, 0], np.array(f["sc"][0]))


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_transpose_identity_with_per_row_quantizer(dtype):
    """Per-channel quantization of x[g] is per-row quantization of x[g]^T."""
    rng = np.random.default_rng(3)
    G, T, d = 3, 57, 48
    x = (rng.standard_normal((G, T, d)) * np.exp(rng.uniform(-6, 6, (G, 1, d)))).astype(dtype)
    x[1, :, 5] = 0                                   # an all-zero channel
    codes, s = OC.quantize_int8_channel(x)
    for g in range(G):
        c_row, s_row = O8.quantize_int8(np.ascontiguousarray(x[g].T))
        assert np.array_equal(s[g].view(np.uint32), s_row.view(np.uint32))
        assert np.array_equal(codes[g], c_row.T)
    xh = OC.dequantize_int8_channel(codes, s)
    for g in range(G):
        want = O8.dequantize_int8(np.ascontiguousarray(codes[g].T), s[g]).T
        assert np.array_equal(xh[g].view(np.uint32), want.view(np.uint32))


def test_exact_rationals():
    rng = np.random.default_rng(4)
    G, T, d = 2, 9, 16
    x = (rng.standard_normal((G, T, d)) * 3).astype(np.float32)
    codes, s = OC.quantize_int8_channel(x)
    q = rng.standard_normal((G, 2, d)).astype(np.float32)
    sig = OC.scores_int8_channel(q, codes, s)
    for g in range(G):
        for c in range(d):
            a = max(abs(Fraction(float(x[g, t, c]))) for t in range(T))
            sc = E.rn32(a / 127)
            assert Fraction(float(s[g, c])) == sc
            for t in range(T):
                want = 0 if sc == 0 else max(-128, min(127, E.round_half_even_int(
                    E.rn32(Fraction(float(x[g, t, c])) / sc))))
                assert int(codes[g, t, c]) == want
        for j in range(2):
            for t in range(T):
                ex = sum(Fraction(float(q[g, j, c])) * Fraction(float(s[g, c])) * int(codes[g, t, c])
                         for c in range(d))
                assert abs(sig[g, j, t] - float(ex)) <= 1e-12 * (1 + abs(float(ex)))


def test_codes_reach_127_in_every_live_channel():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 100, 64)).astype(np.float32)
    codes, s = OC.quantize_int8_channel(x)
    assert np.all(np.abs(codes.astype(np.int32)).max(axis=1) == 127)
    assert codes.min() >= -127
