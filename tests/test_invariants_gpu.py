"""Metamorphic checks on the GPU outputs.

Each test transforms an input in a way whose effect on the output follows
from the definitions alone, runs the library on both inputs and compares the
two outputs; no oracle is involved.  The transformations:

* negation and power-of-two scaling of a row (or of the query), away from
  overflow and underflow: every binary32 / binary16 operation the methods
  use (products, sums, IEEE division, square root, round-half-even) commutes
  with them exactly, so codes and sign bits are unchanged or complemented
  and scales, norms and scores scale or flip bit for bit;
* permutation of tokens (rows), channels or quantization groups: every
  output element depends only on its own token / channel / group;
* degenerate rows: a zero row, an all-equal row, a zero-norm token.

Where a kernel's rounding depends on more than the operands, a check holds
only to the score tolerance (|a - b| <= 1e-5 of the score's magnitude
bound, the bound the parity tests use), and the test says which:
* the matrix-core INT8 scores: power-of-two scaling and token order stay
  exact, negation does not (the dot-product unit's internal rounding is not
  sign-symmetric);
* QJL scores with complemented sign words: the byte tables hold sums of the
  projected query over set bits, so the complement is a different sum;
* token order in the fp16 QJL and two-stage scores: a lane starts its
  sign-byte table reads at the byte given by its token's slot (t mod 32,
  t mod 8), so that the lanes of a wave read different LDS banks; the sum's
  order, and so its rounding, then depends on the slot.

Passages whose definitions fix these outcomes:
* Q-TensorFormer model card, section 6: symmetric INT8 (absmax / 127, round,
  clamp) and asymmetric group-wise INT4 ((max - min) / 15, offset min);
* QJL page, abstract: sign bits of a Gaussian projection of the key, the
  key's norm, and the asymmetric estimator with the query projected
  unquantized;
* TurboQuant news item: QJL of the residual after a coarse quantizer;
* decode: softmax-weighted sum over the tokens, which no token order changes
  beyond fp32 rounding.
"""
import numpy as np
import pytest
import torch

import kv_cache_compression_kvq_amd as K

pytestmark = pytest.mark.gpu

DEV = "cuda"
F = {"f32": torch.float32, "f16": torch.float16}


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def rows_with_spread(R, d, dt, seed, spread):
    """R rows of N(0,1) values, row r multiplied by exp(U(-spread, spread))."""
    g = gen(seed)
    x = torch.randn(R, d, device=DEV, generator=g, dtype=torch.float32)
    x *= torch.exp(torch.empty(R, 1, device=DEV).uniform_(-spread, spread, generator=g))
    return x.to(F[dt])


def same(a: torch.Tensor, b: torch.Tensor, what: str):
    """Bit-for-bit equality (for floats: equal values, +0 == -0)."""
    assert a.shape == b.shape, what
    if a.is_floating_point():
        bad = ~(a == b)
    else:
        bad = a != b
    n = int(bad.sum())
    assert n == 0, f"{what}: {n} of {a.numel()} elements differ"


def perm(T, seed):
    return torch.randperm(T, device=DEV, generator=gen(seed))


def close(a: torch.Tensor, b: torch.Tensor, mag: torch.Tensor, what: str, rel=1e-5):
    """|a - b| <= rel * mag elementwise (mag: the score's magnitude bound)."""
    assert a.shape == b.shape, what
    err = (a.double() - b.double()).abs() / (mag.double() + 1e-300)
    worst = float(err.max()) if err.numel() else 0.0
    assert worst <= rel, f"{what}: {worst:.3g} of the magnitude bound (limit {rel:g})"


def int8_mag(q, codes, scales):
    """s_t sum_i |q_i c_ti|, [G, nq, T], in fp64."""
    a = torch.matmul(q.double().abs(), codes.double().abs().transpose(1, 2).contiguous())
    return a * scales.double()[:, None, :]


def qjl_mag(q, S, norms):
    """sqrt(pi/2) / m * n_t * sum_i |(S q)_i|, [G, nq, T], in fp64."""
    m = S.shape[0]
    y = torch.matmul(q.double(), S.double().t().contiguous()).abs().sum(dim=-1)
    return (np.sqrt(np.pi / 2) / m) * y[:, :, None] * norms.double()[:, None, :]


# ---------------------------------------------------------------- INT8, per token

@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("d", [128, 1024])
def test_int8_quantize_invariants(dt, d):
    R = 2 * 700 + 5
    x = rows_with_spread(R, d, dt, 11 + d, 2.0)
    x[3] = 0
    x[4] = 0.75
    x[5] = -3.0
    codes, scales = K.quantize_int8(x)

    assert int(codes.min()) >= -127 and int(codes.max()) <= 127
    nz = scales != 0
    am = x.float().abs().argmax(dim=1)
    at = codes.gather(1, am[:, None])[:, 0].int()
    xs = x.float().gather(1, am[:, None])[:, 0]
    same(at[nz], (torch.sign(xs[nz]) * 127).int(), "code at the row's absmax")
    assert float(scales[3]) == 0.0 and int(codes[3].abs().max()) == 0
    same(codes[4], torch.full_like(codes[4], 127), "all-equal positive row")
    same(codes[5], torch.full_like(codes[5], -127), "all-equal negative row")

    c2, s2 = K.quantize_int8(-x)
    same(c2, -codes, "codes of -x")
    same(s2, scales, "scales of -x")
    for f in ((8.0, 0.0625) if dt == "f32" else (8.0,)):
        c2, s2 = K.quantize_int8(x * f)
        same(c2, codes, f"codes of {f} x")
        same(s2, scales * f, f"scales of {f} x")
    p = perm(R, 3)
    c2, s2 = K.quantize_int8(x[p])
    same(c2, codes[p], "codes of permuted rows")
    same(s2, scales[p], "scales of permuted rows")

    v = K.dequantize_int8(codes, scales)
    same(K.dequantize_int8(-codes, scales), -v, "dequantized -codes")
    same(K.dequantize_int8(codes, scales * 8), v * 8, "dequantized with 8 s")


@pytest.mark.parametrize("qdt", ["f32", "f16"])
@pytest.mark.parametrize("nq,d", [(1, 128), (2, 128), (3, 128), (4, 128), (8, 128), (1, 64),
                                  (3, 96)])
def test_int8_scores_linear_and_permutation(qdt, nq, d):
    G, T = 3, 1029
    g = gen(nq * 100 + d)
    codes = torch.randint(-127, 128, (G, T, d), device=DEV, generator=g, dtype=torch.int8)
    scales = torch.empty(G, T, device=DEV).uniform_(1e-3, 5e-2, generator=g)
    scales[:, ::97] = 0
    q = torch.randn(G, nq, d, device=DEV, generator=g).to(F[qdt])
    sc = K.scores_int8(q, codes, scales)
    mfma = d == 128 and 4 <= nq <= (16 if qdt == "f16" else 8)
    if mfma:
        close(K.scores_int8(-q, codes, scales), -sc, int8_mag(q, codes, scales), "scores of -q")
    else:
        same(K.scores_int8(-q, codes, scales), -sc, "scores of -q")
    same(K.scores_int8(q * 4, codes, scales), sc * 4, "scores of 4 q")
    assert not bool(sc[:, :, ::97].any()), "a token with scale 0 scored non-zero"
    p = perm(T, nq)
    same(K.scores_int8(q, codes[:, p], scales[:, p]), sc[:, :, p], "scores of permuted tokens")


# ---------------------------------------------------------------- INT8, per channel

@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("T", [1000, 5003])
def test_int8_channel_invariants(dt, T):
    G, d = 2, 128
    g = gen(T)
    x = torch.randn(G, T, d, device=DEV, generator=g)
    x *= torch.exp(torch.empty(G, 1, d, device=DEV).uniform_(-2, 2, generator=g))
    x = x.to(F[dt])
    codes, scales = K.quantize_int8_channel(x)

    c2, s2 = K.quantize_int8_channel(-x)
    same(c2, -codes, "codes of -x")
    same(s2, scales, "scales of -x")
    x2 = x.clone()
    x2[:, :, 17] *= 8
    c2, s2 = K.quantize_int8_channel(x2)
    same(c2, codes, "codes with channel 17 scaled by 8")
    want = scales.clone()
    want[:, 17] *= 8
    same(s2, want, "scales with channel 17 scaled by 8")
    p = perm(T, 5)
    c2, s2 = K.quantize_int8_channel(x[:, p])
    same(c2, codes[:, p], "codes of permuted tokens")
    same(s2, scales, "scales of permuted tokens")
    pc = perm(d, 6)
    c2, s2 = K.quantize_int8_channel(x[:, :, pc])
    same(c2, codes[:, :, pc], "codes of permuted channels")
    same(s2, scales[:, pc], "scales of permuted channels")

    for nq in (1, 4):
        q = torch.randn(G, nq, d, device=DEV, generator=g).to(F[dt])
        sc = K.scores_int8_channel(q, codes, scales)
        if nq == 1:
            same(K.scores_int8_channel(-q, codes, scales), -sc, f"nq {nq}: scores of -q")
        else:
            mag = int8_mag(q.float() * scales[:, None, :], codes, torch.ones_like(codes[..., 0],
                                                                               dtype=torch.float32))
            close(K.scores_int8_channel(-q, codes, scales), -sc, mag, f"nq {nq}: scores of -q")
        same(K.scores_int8_channel(q * 4, codes, scales), sc * 4, f"nq {nq}: scores of 4 q")
        same(K.scores_int8_channel(q, codes[:, p], scales), sc[:, :, p],
             f"nq {nq}: scores of permuted tokens")


# ---------------------------------------------------------------- INT4

@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("d,g", [(128, 32), (128, 128), (256, 64)])
def test_int4_invariants(dt, d, g):
    R = 3 * 512 + 9
    x = rows_with_spread(R, d, dt, d + g, 2.0)
    x[7] = 1.25
    codes, steps, offsets = K.quantize_int4(x, g)
    assert float(steps[7].abs().max()) == 0.0 and int(codes[7].max()) == 0

    for f in ((8.0, 0.0625) if dt == "f32" else (8.0,)):
        c2, s2, o2 = K.quantize_int4(x * f, g)
        same(c2, codes, f"codes of {f} x")
        same(s2, steps * f, f"steps of {f} x")
        same(o2, offsets * f, f"offsets of {f} x")
    p = perm(R, 7)
    c2, s2, o2 = K.quantize_int4(x[p], g)
    same(c2, codes[p], "codes of permuted rows")
    same(s2, steps[p], "steps of permuted rows")
    same(o2, offsets[p], "offsets of permuted rows")
    ng = d // g
    pg = perm(ng, 8)
    xg = x.reshape(R, ng, g)[:, pg].reshape(R, d)
    c2, s2, o2 = K.quantize_int4(xg, g)
    same(c2, codes.reshape(R, ng, g // 2)[:, pg].reshape(R, d // 2), "codes of permuted groups")
    same(s2, steps[:, pg], "steps of permuted groups")
    same(o2, offsets[:, pg], "offsets of permuted groups")
    v = K.dequantize_int4(codes, steps, offsets, g)
    same(K.dequantize_int4(codes, steps * 8, offsets * 8, g), v * 8, "dequantized, 8 s and 8 z")


# ---------------------------------------------------------------- QJL

@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("d,m", [(128, 256), (64, 128), (128, 512), (96, 64)])
def test_qjl_sketch_invariants(dt, d, m):
    R = 2 * 1500 + 7
    g = gen(d * m)
    S = torch.randn(m, d, device=DEV, generator=g).to(F[dt])
    k = rows_with_spread(R, d, dt, d + m, 1.0)
    k[9] = 0
    bits, norms = K.qjl_sketch(k, S)
    same(bits[9], torch.full_like(bits[9], -1), "sign words of a zero key")
    assert float(norms[9]) == 0.0

    b2, n2 = K.qjl_sketch(-k, S)
    live = torch.ones(R, dtype=torch.bool, device=DEV)
    live[9] = False
    same(b2[live], ~bits[live], "sign words of -k")
    same(n2, norms, "norms of -k")
    for f in ((8.0, 0.0625) if dt == "f32" else (8.0,)):
        b2, n2 = K.qjl_sketch(k * f, S)
        same(b2, bits, f"sign words of {f} k")
        same(n2, (norms.float() * f).half(), f"norms of {f} k")
    p = perm(R, 9)
    b2, n2 = K.qjl_sketch(k[p], S)
    same(b2, bits[p], "sign words of permuted rows")
    same(n2, norms[p], "norms of permuted rows")


@pytest.mark.parametrize("qdt", ["f32", "f16"])
@pytest.mark.parametrize("nq,T", [(1, 1500), (1, 5000), (4, 1500), (4, 5000), (3, 777)])
def test_qjl_scores_linear_and_permutation(qdt, nq, T):
    G, d, m = 3, 128, 256
    g = gen(nq * 10 + T)
    S = torch.randn(m, d, device=DEV, generator=g).to(F[qdt])
    bits = torch.randint(-2**31, 2**31 - 1, (G, T, m // 32), device=DEV, generator=g,
                         dtype=torch.int32)
    norms = torch.empty(G, T, device=DEV).uniform_(0.5, 4.0, generator=g).half()
    norms[:, ::89] = 0
    q = torch.randn(G, nq, d, device=DEV, generator=g).to(F[qdt])
    sc = K.scores_qjl(q, S, bits, norms)
    # 2 .. 8 queries with fp16 S run on the matrix cores, whose accumulation
    # is not symmetric under negation; the byte-table kernels' is
    if qdt == "f16" and 2 <= nq <= 8:
        close(K.scores_qjl(-q, S, bits, norms), -sc, qjl_mag(q, S, norms), "scores of -q")
    else:
        same(K.scores_qjl(-q, S, bits, norms), -sc, "scores of -q")
    same(K.scores_qjl(q * 4, S, bits, norms), sc * 4, "scores of 4 q")
    close(K.scores_qjl(q, S, ~bits, norms), -sc, qjl_mag(q, S, norms),
          "scores of complemented sign words")
    assert not bool(sc[:, :, ::89].any()), "a zero-norm token scored non-zero"
    p = perm(T, 11)
    sp = K.scores_qjl(q, S, bits[:, p], norms[:, p])
    if qdt == "f32":
        same(sp, sc[:, :, p], "scores of permuted tokens")
    else:
        close(sp, sc[:, :, p], qjl_mag(q, S, norms)[:, :, p], "scores of permuted tokens")


# ---------------------------------------------------------------- two-stage (INT4 + residual QJL)

@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("g", [32, 128])
def test_residual_invariants(dt, g):
    G, T, d, m = 2, 1300, 128, 256
    gg = gen(g)
    S = torch.randn(m, d, device=DEV, generator=gg).to(F[dt])
    k = rows_with_spread(G * T, d, dt, 40 + g, 1.0).reshape(G, T, d)
    out = K.residual_sketch(k, S, g)
    names = ("codes", "steps", "offsets", "sign words", "norms")

    o2 = K.residual_sketch(k * 8, S, g)
    for a, b, nm in zip(out, o2, names):
        if nm in ("codes", "sign words"):
            same(b, a, f"{nm} of 8 k")
        elif nm == "norms":
            same(b, (a.float() * 8).half(), f"{nm} of 8 k")
        else:
            same(b, a * 8, f"{nm} of 8 k")
    p = perm(T, 12)
    o2 = K.residual_sketch(k[:, p], S, g)
    for a, b, nm in zip(out, o2, names):
        same(b, a[:, p], f"{nm} of permuted tokens")

    for nq in (1, 4):
        q = torch.randn(G, nq, d, device=DEV, generator=gg).to(F[dt])
        sc = K.scores_residual(q, S, *out, g)
        same(K.scores_residual(-q, S, *out, g), -sc, f"nq {nq}: scores of -q")
        same(K.scores_residual(q * 4, S, *out, g), sc * 4, f"nq {nq}: scores of 4 q")
        sp = K.scores_residual(q, S, *(t[:, p] for t in out), g)
        if dt == "f32":
            same(sp, sc[:, :, p], f"nq {nq}: scores of permuted tokens")
        else:
            khat = K.dequantize_int4(out[0], out[1], out[2], g)
            mag = int8_mag(q, khat, torch.ones_like(out[4], dtype=torch.float32))
            mag = mag + qjl_mag(q, S, out[4])
            close(sp, sc[:, :, p], mag[:, :, p], f"nq {nq}: scores of permuted tokens")


# ---------------------------------------------------------------- decode

def decode_cache(G, T, d, m, seed):
    g = gen(seed)
    S = torch.randn(m, d, device=DEV, generator=g).half()
    kbits = torch.randint(-2**31, 2**31 - 1, (G, T, m // 32), device=DEV, generator=g,
                          dtype=torch.int32)
    knorms = torch.empty(G, T, device=DEV).uniform_(0.5, 2.0, generator=g).half()
    vcodes = torch.randint(-127, 128, (G, T, d), device=DEV, generator=g, dtype=torch.int8)
    vscales = torch.empty(G, T, device=DEV).uniform_(1e-3, 5e-2, generator=g)
    return g, S, kbits, knorms, vcodes, vscales


def vhat_bound(vcodes, vscales):
    """max_t |c_t s_t| per (group, channel): the scale of a decode output."""
    return (vcodes.float() * vscales[..., None]).abs().amax(dim=-2)


@pytest.mark.parametrize("T", [1, 777, 20000])
def test_decode_token_order_and_value_scaling(T):
    G, d, m = 4, 128, 256
    g, S, kbits, knorms, vcodes, vscales = decode_cache(G, T, d, m, T)
    q = torch.randn(G, d, device=DEV, generator=g).half()
    out = K.decode_qjl_int8(q, S, kbits, knorms, vcodes, vscales)
    bound = vhat_bound(vcodes, vscales)
    if T == 1:
        v0 = vcodes[:, 0].float() * vscales[:, :1]
        assert bool(((out - v0).abs() <= 1e-6 * bound + 1e-30).all()), "T = 1 is not v_0"
    p = perm(T, 13)
    o2 = K.decode_qjl_int8(q, S, kbits[:, p], knorms[:, p], vcodes[:, p], vscales[:, p])
    err = float(((o2 - out).abs() / (bound + 1e-30)).max())
    assert err <= 1e-5, f"permuted tokens moved the output by {err:.3g} of max |v|"
    same(K.decode_qjl_int8(q, S, kbits, knorms, vcodes, vscales * 8), out * 8,
         "output with 8 v-scales")


@pytest.mark.parametrize("T", [300, 9000])
def test_decode_equal_keys_give_the_value_mean(T):
    G, d, m = 3, 128, 256
    g, S, kbits, knorms, vcodes, vscales = decode_cache(G, T, d, m, 50 + T)
    kbits[:] = kbits[:, :1]
    knorms[:] = knorms[:, :1]
    q = torch.randn(G, d, device=DEV, generator=g).half()
    out = K.decode_qjl_int8(q, S, kbits, knorms, vcodes, vscales)
    mean = (vcodes.double() * vscales.double()[..., None]).mean(dim=1)
    err = float(((out.double() - mean).abs() / (vhat_bound(vcodes, vscales).double() + 1e-30)).max())
    assert err <= 1e-5, f"equal keys: output {err:.3g} of max |v| away from the value mean"


@pytest.mark.parametrize("nq,T", [(4, 3000), (8, 20000), (3, 515)])
def test_decode_grouped_query_and_token_order(nq, T):
    G, d, m = 4, 128, 256
    g, S, kbits, knorms, vcodes, vscales = decode_cache(G, T, d, m, nq * T)
    q = torch.randn(G, nq, d, device=DEV, generator=g).half()
    out = K.decode_qjl_int8_gqa(q, S, kbits, knorms, vcodes, vscales)
    bound = vhat_bound(vcodes, vscales)[:, None, :]
    pq = perm(nq, 14)
    o2 = K.decode_qjl_int8_gqa(q[:, pq], S, kbits, knorms, vcodes, vscales)
    err = float(((o2 - out[:, pq]).abs() / (bound + 1e-30)).max())
    assert err <= 1e-5, f"permuted queries moved the output by {err:.3g} of max |v|"
    p = perm(T, 15)
    o2 = K.decode_qjl_int8_gqa(q, S, kbits[:, p], knorms[:, p], vcodes[:, p], vscales[:, p])
    err = float(((o2 - out).abs() / (bound + 1e-30)).max())
    assert err <= 1e-5, f"permuted tokens moved the output by {err:.3g} of max |v|"
    o2 = K.decode_qjl_int8_gqa(q, S, kbits, knorms, vcodes, vscales * 8)
    err = float(((o2 - out * 8).abs() / (8 * bound + 1e-30)).max())
    assert err <= 1e-6, f"8 v-scales: output off 8 x by {err:.3g} of max |v|"
