"""GPU parity of the fused decode step (QJL keys, INT8 values, softmax)
against the oracle: |o_j - o_j^ora| <= 1e-4 * sum_t p_t |v_hat_tj| + 1e-6,
given identical compressed inputs (made by the oracle and uploaded)."""
import math

import numpy as np
import pytest
import torch

import kv_cache_compression_kvq_amd as K
import synth_inputs as si
from oracle import decode as OD, int8 as OI, qjl as OQ
import full_size as FS
from gpu_common import (assert_bits_within_band, assert_norms_within_ulp, decode_tolerance_check,
                        down, log, up)

pytestmark = pytest.mark.gpu


def make_cache(k, v, S):
    """Oracle-made compressed cache for keys k [G, T, d] and values v."""
    G, T, d = k.shape
    kw, kn = OQ.qjl_sketch(k.reshape(-1, d), S)
    vc, vs = OI.quantize_int8(v.reshape(-1, d))
    m = S.shape[0]
    return kw.reshape(G, T, m // 32), kn.reshape(G, T), vc.reshape(G, T, d), vs.reshape(G, T)


def decode_check(q, S, kw, kn, vc, vs, lam, label):
    log(f"[decode] {label}: G={q.shape[0]} T={kw.shape[1]} d={q.shape[1]} m={S.shape[0]}")
    out = down(K.decode_qjl_int8(up(q), up(S), up(kw), up(kn), up(vc), up(vs), lam))
    ora = OD.decode_qjl_int8(q, S, kw, kn, vc, vs, lam)
    worst = decode_tolerance_check(out, q, S, kw, kn, vc, vs, lam, ora)
    log(f"[decode] {label}: worst err / tol = {worst:.3g}")
    return out


def test_tiny_decode():
    W = si.W_TINY
    k = si.kv_tensor(W, si.K, 1, 1, 512, 128, "f32").reshape(1, 512, 128)
    v = si.kv_tensor(W, si.V, 1, 1, 512, 128, "f32").reshape(1, 512, 128)
    S = si.projection(W, 256, 128, "f32")
    q = si.queries(W, 1, 1, 128, "f32")[:, 0]
    decode_check(q, S, *make_cache(k, v, S), 1 / math.sqrt(128), "tiny")


@pytest.mark.parametrize("G,T", [(2, 1), (3, 63), (4, 257), (16, 5000), (1, 40000)])
def test_decode_shapes_fp16(G, T):
    W = si.W_DECODE
    d, m = 128, 256
    k = si.kv_tensor(W, si.K, 1, G, T, d, "f16").reshape(G, T, d)
    v = si.kv_tensor(W, si.V, 1, G, T, d, "f16").reshape(G, T, d)
    S = si.projection(W, m, d, "f16")
    q = si.queries(W, G, 1, d, "f16")[:, 0]
    decode_check(q, S, *make_cache(k, v, S), 1 / math.sqrt(d), f"G={G} T={T}")


@pytest.mark.parametrize("d,m,qdt", [(64, 256, "f16"), (256, 256, "f32"), (96, 128, "f16"),
                                     (128, 512, "f32"), (128, 64, "f16"), (16, 32, "f32")])
def test_decode_other_shapes(d, m, qdt):
    rng = np.random.default_rng(d + m)
    G, T = 5, 777
    npq = np.float16 if qdt == "f16" else np.float32
    k = rng.standard_normal((G, T, d)).astype(np.float16)
    v = rng.standard_normal((G, T, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(npq)
    q = rng.standard_normal((G, d)).astype(npq)
    decode_check(q, S, *make_cache(k, v, S), 1 / math.sqrt(d), f"d={d} m={m} q={qdt}")


def test_single_token_returns_its_value_exactly_enough():
    rng = np.random.default_rng(3)
    G, d, m = 4, 128, 256
    k = rng.standard_normal((G, 1, d)).astype(np.float16)
    v = rng.standard_normal((G, 1, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(np.float16)
    q = rng.standard_normal((G, d)).astype(np.float16)
    kw, kn, vc, vs = make_cache(k, v, S)
    out = down(K.decode_qjl_int8(up(q), up(S), up(kw), up(kn), up(vc), up(vs), 0.1))
    want = vc[:, 0].astype(np.float64) * vs[:, 0, None]
    assert np.allclose(out, want, rtol=1e-6, atol=0)


def test_split_invariance():
    """The same group decoded alone (many splits) and among many groups
    (fewer splits) gives the same output up to binary32 rounding."""
    rng = np.random.default_rng(9)
    d, m, T = 128, 256, 20000
    G = 600
    S = rng.standard_normal((m, d)).astype(np.float16)
    k = rng.standard_normal((2, T, d)).astype(np.float16)
    v = rng.standard_normal((2, T, d)).astype(np.float16)
    kw, kn, vc, vs = make_cache(k, v, S)
    q = rng.standard_normal((2, d)).astype(np.float16)
    alone = down(K.decode_qjl_int8(up(q[:1]), up(S), up(kw[:1]), up(kn[:1]), up(vc[:1]), up(vs[:1])))
    rep = lambda a: np.ascontiguousarray(np.repeat(a[:1], G, axis=0))
    many = down(K.decode_qjl_int8(up(rep(q)), up(S), up(rep(kw)), up(rep(kn)), up(rep(vc)), up(rep(vs))))
    assert K.decode_workspace_bytes(1, T, d, m) // (d + 2) // 4 != K.decode_workspace_bytes(G, T, d, m) // G // (d + 2) // 4
    assert np.allclose(many, alone[0][None, :], rtol=2e-5, atol=1e-6)


def test_decode_full_size_every_group():
    """16 x 32 x 32768 x 128: K sketched and V quantized on the GPU from the
    generator's fp16 tensors; every row of that cache is checked against the
    oracle (sign bits within the band, norms within one ulp, value codes and
    scales bit-exact).  The full-size decode (the bench's launch) then runs
    on the GPU-built cache, and the oracle, fed the same cache, checks the
    output of every one of the 512 groups; then the grouped-query decode of
    4 queries for each of the first 128 heads (the bench's grouped shape),
    every (head, query) output."""
    W = si.W_DECODE
    B, H, T, d, m = 16, 32, 32768, 128, 256
    G = B * H
    lam = 1 / math.sqrt(d)
    log("[decode] full size: generate K")
    k = si.kv_tensor(W, si.K, B, H, T, d, "f16").reshape(G * T, d)
    S = si.projection(W, m, d, "f16")
    Sd = up(S)
    kd = up(k)
    kbits, knorms = K.qjl_sketch(kd, Sd)
    del kd
    kw, kn = down(kbits, np.uint32), down(knorms)
    log("[decode] full size: check every key row")
    flips, ulps = FS.sketch_every_row(k, S, kw, kn)
    log(f"[decode] full size: {flips} key bits inside the band differ, {ulps} norms one ulp apart")
    del k
    log("[decode] full size: generate V")
    v = si.kv_tensor(W, si.V, B, H, T, d, "f16").reshape(G * T, d)
    vd = up(v)
    vcodes, vscales = K.quantize_int8(vd)
    del vd
    vc, vs = down(vcodes), down(vscales)
    log("[decode] full size: check every value row")
    FS.int8_every_row(v, vc, vs, K.dequantize_int8(vcodes, vscales, torch.float16).cpu().numpy(),
                      "decode V", out_dtype="f16")
    del v
    q = si.queries(W, G, 1, d, "f16")[:, 0]
    log("[decode] full size: decode")
    out = down(K.decode_qjl_int8(up(q), Sd, kbits.view(G, T, m // 32), knorms.view(G, T),
                                 vcodes.view(G, T, d), vscales.view(G, T), lam))
    assert np.all(np.isfinite(out))
    log("[decode] full size: oracle on every group")
    worst = FS.decode_every_group(q, S, kw.reshape(G, T, m // 32), kn.reshape(G, T),
                                  vc.reshape(G, T, d), vs.reshape(G, T), lam, out)
    log(f"[decode] full size: all {G} groups within tolerance; worst err / tol = {worst:.3g}")
    # grouped-query decode at the bench's grouped shape on the same cache:
    # 128 KV heads x 32768 tokens, 4 queries per head, every (head, query)
    Gk, nq = 128, 4
    q4 = si.queries(W, Gk, nq, d, "f16")
    log("[decode] full size: grouped decode, 128 KV heads x 4 queries")
    out4 = down(K.decode_qjl_int8_gqa(up(q4), Sd, kbits.view(G, T, m // 32)[:Gk],
                                      knorms.view(G, T)[:Gk], vcodes.view(G, T, d)[:Gk],
                                      vscales.view(G, T)[:Gk], lam))
    assert np.all(np.isfinite(out4))
    for j in range(nq):
        worst = FS.decode_every_group(np.ascontiguousarray(q4[:, j]), S, kw.reshape(G, T, m // 32)[:Gk],
                                      kn.reshape(G, T)[:Gk], vc.reshape(G, T, d)[:Gk],
                                      vs.reshape(G, T)[:Gk], lam, np.ascontiguousarray(out4[:, j]))
        log(f"[decode] full size: grouped query {j}: all {Gk} heads within tolerance; "
            f"worst err / tol = {worst:.3g}")


# --- grouped-query attention: nq query heads per KV head -------------------------

@pytest.mark.parametrize("G,nq,T,d,m", [(2, 4, 3000, 128, 256), (3, 2, 257, 128, 256), (1, 8, 5000, 128, 256),
                                        (4, 3, 700, 64, 128), (2, 5, 63, 256, 256), (8, 4, 1, 128, 256)])
def test_decode_grouped_queries(G, nq, T, d, m):
    """Each of a group's nq queries gets what the oracle's decode gives for it
    alone (every query checked against the one-query definition)."""
    rng = np.random.default_rng(G * 100 + nq * 10 + T)
    k = rng.standard_normal((G, T, d)).astype(np.float16)
    v = rng.standard_normal((G, T, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(np.float16)
    kw, kn, vc, vs = make_cache(k, v, S)
    q = rng.standard_normal((G, nq, d)).astype(np.float16)
    lam = 1 / math.sqrt(d)
    log(f"[decode-gqa] G={G} nq={nq} T={T} d={d} m={m}")
    out = down(K.decode_qjl_int8_gqa(up(q), up(S), up(kw), up(kn), up(vc), up(vs), lam))
    assert out.shape == (G, nq, d)
    worst = 0.0
    for j in range(nq):
        qj = np.ascontiguousarray(q[:, j])
        ora = OD.decode_qjl_int8(qj, S, kw, kn, vc, vs, lam)
        worst = max(worst, decode_tolerance_check(out[:, j], qj, S, kw, kn, vc, vs, lam, ora))
    log(f"[decode-gqa] worst err / tol = {worst:.3g}")


@pytest.mark.parametrize("G,nq,T,qscale", [(3, 2, 1000, 1.0), (2, 3, 2049, 1.0), (2, 4, 8191, 1.0),
                                           (1, 5, 3000, 1.0), (2, 6, 700, 1.0), (300, 4, 513, 1.0),
                                           (1, 4, 70001, 1.0), (4, 4, 4096, 8.0), (5, 7, 1, 1.0)])
def test_decode_grouped_one_pass(G, nq, T, qscale):
    """d = 128, m = 256: one pass over each token range carries up to four
    query heads (three: one zero-table slot; five to seven: a pass of four and
    one of the rest); every query is checked against the oracle's one-query
    decode.  qscale > 1 makes the softmax peaky (a few tokens carry it)."""
    rng = np.random.default_rng(G * 1000 + nq * 100 + T % 97)
    d, m = 128, 256
    k = rng.standard_normal((G, T, d)).astype(np.float16)
    v = rng.standard_normal((G, T, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(np.float16)
    kw, kn, vc, vs = make_cache(k, v, S)
    q = (rng.standard_normal((G, nq, d)) * qscale).astype(np.float16)
    lam = 1 / math.sqrt(d)
    log(f"[decode-gqa1] G={G} nq={nq} T={T} qscale={qscale}")
    out = down(K.decode_qjl_int8_gqa(up(q), up(S), up(kw), up(kn), up(vc), up(vs), lam))
    worst = 0.0
    for j in range(nq):
        qj = np.ascontiguousarray(q[:, j])
        ora = OD.decode_qjl_int8(qj, S, kw, kn, vc, vs, lam)
        worst = max(worst, decode_tolerance_check(out[:, j], qj, S, kw, kn, vc, vs, lam, ora))
    log(f"[decode-gqa1] worst err / tol = {worst:.3g}")


@pytest.mark.parametrize("pattern", ["rising", "falling", "scattered", "zeros"])
def test_decode_grouped_value_scales_across_binades(pattern):
    """The one-pass grouped decode sums the values on the matrix cores with
    binary16 weights scaled by a running power of two (from the largest value
    scale seen): value scales spanning 2^-40 .. 2^40 that grow along the
    range (rescaling mid-range), shrink, scatter, or include all-zero value
    rows; every query checked against the oracle."""
    rng = np.random.default_rng(len(pattern) * 31)
    G, nq, T, d, m = 3, 4, 3001, 128, 256
    k = rng.standard_normal((G, T, d)).astype(np.float16)
    v = rng.standard_normal((G, T, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(np.float16)
    kw, kn, vc, vs = make_cache(k, v, S)
    ramp = np.linspace(-40.0, 40.0, T)
    expo = {"rising": ramp, "falling": -ramp, "scattered": rng.uniform(-40, 40, T),
            "zeros": rng.uniform(-3, 3, T)}[pattern]
    vs = (np.exp2(expo)[None, :] * rng.uniform(0.5, 1.0, (G, T))).astype(np.float32)
    if pattern == "zeros":
        vs[:, rng.integers(0, T, T // 3)] = 0.0
        vs[1] = 0.0                                    # a head whose values are all zero
    q = (rng.standard_normal((G, nq, d)) * 2.0).astype(np.float16)
    lam = 1 / math.sqrt(d)
    log(f"[decode-gqa-binades] {pattern}")
    out = down(K.decode_qjl_int8_gqa(up(q), up(S), up(kw), up(kn), up(vc), up(vs), lam))
    worst = 0.0
    for j in range(nq):
        qj = np.ascontiguousarray(q[:, j])
        ora = OD.decode_qjl_int8(qj, S, kw, kn, vc, vs, lam)
        worst = max(worst, decode_tolerance_check(out[:, j], qj, S, kw, kn, vc, vs, lam, ora))
    log(f"[decode-gqa-binades] {pattern}: worst err / tol = {worst:.3g}")


def test_decode_grouped_single_query_equals_plain_decode():
    """nq = 1 through the grouped entry point is the plain decode, bit for bit."""
    rng = np.random.default_rng(77)
    G, T, d, m = 5, 3000, 128, 256
    k = rng.standard_normal((G, T, d)).astype(np.float16)
    v = rng.standard_normal((G, T, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(np.float16)
    kw, kn, vc, vs = (up(a) for a in make_cache(k, v, S))
    q = rng.standard_normal((G, 1, d)).astype(np.float16)
    a = down(K.decode_qjl_int8_gqa(up(q), up(S), kw, kn, vc, vs))
    b = down(K.decode_qjl_int8(up(np.ascontiguousarray(q[:, 0])), up(S), kw, kn, vc, vs))
    assert np.array_equal(a[:, 0].view(np.uint32), b.view(np.uint32))
