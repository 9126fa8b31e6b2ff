"""Whole-output comparisons of full-size GPU results with the oracle (test
code only).

The oracle runs on every row / group, cut into chunks that a thread pool
processes in parallel (numpy releases the GIL inside its array operations),
so a 2^30-element or 16.8M-token output is checked in seconds to minutes of
host time.  Each function takes host copies of the GPU's outputs and raises
AssertionError naming the first offending row or group.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import decode as OD, int8 as OI, qjl as OQ


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool_map(fn, items):
    with ThreadPoolExecutor(max_workers=workers()) as ex:
        return list(ex.map(fn, items))


def _chunks(n: int, size: int):
    return [(a, min(n, a + size)) for a in range(0, n, size)]


def int8_every_row(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, deq: np.ndarray,
                   label: str, out_dtype: str = "f32") -> None:
    """Codes, scales and dequantised values of every row of x [R, d] equal the
    oracle's bit for bit."""
    R, d = x.shape
    u = np.uint16 if out_dtype == "f16" else np.uint32

    def one(span):
        a, b = span
        co, so = OI.quantize_int8(x[a:b])
        if not np.array_equal(scales[a:b].view(np.uint32), so.view(np.uint32)):
            r = a + int(np.nonzero(scales[a:b].view(np.uint32) != so.view(np.uint32))[0][0])
            return f"{label}: scale of row {r} differs"
        if not np.array_equal(codes[a:b], co):
            r, c = np.nonzero(codes[a:b] != co)
            return f"{label}: {len(r)} codes differ, first at row {a + r[0]} col {c[0]}"
        do = OI.dequantize_int8(co, so, out_dtype)
        if not np.array_equal(deq[a:b].view(u), do.view(u)):
            return f"{label}: dequantised values differ in rows [{a}, {b})"
        return None

    errs = [e for e in _pool_map(one, _chunks(R, max(1, (1 << 21) // d))) if e]
    assert not errs, errs[0]


def sketch_every_row(k: np.ndarray, S: np.ndarray, words: np.ndarray,
                     norms: np.ndarray) -> tuple[int, int]:
    """Sign words of every row of k [R, d] equal the oracle's except for bits
    whose projection lies inside the band |P_ri| <= 1e-4 ||S_i|| ||k_r||;
    norms within one binary16 ulp.  Returns (differing bits, norms off by one
    ulp)."""
    R, d = k.shape
    m = S.shape[0]
    words = words.reshape(R, m // 32)
    norms = norms.reshape(R)
    s_norm = np.linalg.norm(S.astype(np.float64), axis=1)

    def one(span):
        a, b = span
        P = OQ.project(k[a:b], S)                          # [rows, m] fp64
        wo = OQ.pack_signs(P >= 0.0)
        flips = 0
        bad = np.nonzero((words[a:b] != wo).any(axis=1))[0]
        if len(bad):
            gb = OQ.unpack_signs(words[a:b][bad], m)
            ob = OQ.unpack_signs(wo[bad], m)
            kn = np.linalg.norm(k[a:b][bad].astype(np.float64), axis=1)
            band = 1e-4 * kn[:, None] * s_norm[None, :]
            diff = gb != ob
            outside = diff & (np.abs(P[bad]) > band)
            if outside.any():
                r = a + int(bad[np.nonzero(outside.any(axis=1))[0][0]])
                return f"sign bits of row {r} differ outside the 1e-4 band", 0, 0
            flips = int(diff.sum())
        no = OQ.key_norms(k[a:b]).view(np.uint16).astype(np.int64)
        ng = norms[a:b].view(np.uint16).astype(np.int64)
        if np.any(np.abs(no - ng) > 1):
            r = a + int(np.nonzero(np.abs(no - ng) > 1)[0][0])
            return f"norm of row {r} differs by more than one binary16 ulp", 0, 0
        return None, flips, int((no != ng).sum())

    res = _pool_map(one, _chunks(R, 1 << 15))
    errs = [e for e, _, _ in res if e]
    assert not errs, errs[0]
    return sum(f for _, f, _ in res), sum(n for _, _, n in res)


def qjl_scores_every_group(q: np.ndarray, S: np.ndarray, words: np.ndarray, norms: np.ndarray,
                           scores: np.ndarray) -> float:
    """|gpu - ora| <= 1e-4 ||q|| n_t for every score of q [G, nq, d] against
    words [G, T, m / 32] and norms [G, T]; returns the worst err / tol."""
    G = q.shape[0]

    def one(span):
        a, b = span
        ora = OQ.scores_qjl(q[a:b], S, words[a:b], norms[a:b])
        qn = np.linalg.norm(q[a:b].astype(np.float64), axis=-1)
        tol = 1e-4 * qn[:, :, None] * norms[a:b].astype(np.float64)[:, None, :]
        err = np.abs(scores[a:b].astype(np.float64) - ora)
        if np.any(err > tol):
            g = a + int(np.nonzero((err > tol).any(axis=(1, 2)))[0][0])
            return f"QJL scores of group {g} outside 1e-4 ||q|| n_t", 0.0
        return None, float(np.max(err / (tol + 1e-300)))

    res = _pool_map(one, _chunks(G, 4))
    errs = [e for e, _ in res if e]
    assert not errs, errs[0]
    return max(w for _, w in res)


def decode_every_group(q: np.ndarray, S: np.ndarray, kw: np.ndarray, kn: np.ndarray,
                       vc: np.ndarray, vs: np.ndarray, lam: float, out: np.ndarray) -> float:
    """|o_j - o_j^ora| <= 1e-4 sum_t p_t |v_hat_tj| + 1e-6 for every group of
    the decode (q [G, d], cache [G, T, ...]); returns the worst err / tol."""
    G = q.shape[0]
    lam32 = np.float64(np.float32(lam))

    def one(g):
        sig = OQ.scores_qjl(q[g:g + 1, None, :], S, kw[g:g + 1], kn[g:g + 1])[:, 0, :]
        ora = OD.attention(sig, vc[g:g + 1], vs[g:g + 1], lam)
        z = lam32 * sig
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        mag = p @ (np.abs(vc[g].astype(np.float64)) * vs[g].astype(np.float64)[:, None])
        tol = 1e-4 * mag + 1e-6
        err = np.abs(out[g:g + 1].astype(np.float64) - ora)
        if np.any(err > tol):
            return f"decode output of group {g} outside tolerance (max err/tol " \
                   f"{np.max(err / tol):.3g})", 0.0
        return None, float(np.max(err / tol))

    res = _pool_map(one, range(G))
    errs = [e for e, _ in res if e]
    assert not errs, errs[0]
    return max(w for _, w in res)


def int4_every_row(x: np.ndarray, g: int, codes: np.ndarray, steps: np.ndarray,
                   offsets: np.ndarray, deq: np.ndarray, label: str,
                   out_dtype: str = "f32") -> None:
    """INT4 codes, steps and reconstruction of every row of x [R, d] equal the
    oracle's bit for bit; offsets equal by value (a zero offset's sign is
    open) and bit for bit otherwise."""
    from oracle import int4 as O4
    R, d = x.shape
    u = np.uint16 if out_dtype == "f16" else np.uint32

    def one(span):
        a, b = span
        co, so, zo = O4.quantize_int4(x[a:b], g)
        if not np.array_equal(steps[a:b].view(np.uint32), so.view(np.uint32)):
            return f"{label}: steps differ in rows [{a}, {b})"
        zg = offsets[a:b]
        nz = zo != 0
        if not (np.array_equal(zg, zo) and np.array_equal(zg[nz].view(np.uint32),
                                                          zo[nz].view(np.uint32))):
            return f"{label}: offsets differ in rows [{a}, {b})"
        if not np.array_equal(codes[a:b], co):
            r, c = np.nonzero(codes[a:b] != co)
            return f"{label}: {len(r)} code bytes differ, first at row {a + r[0]} byte {c[0]}"
        do = O4.dequantize_int4(co, so, zo, g, out_dtype)
        if not np.array_equal(deq[a:b].view(u), do.view(u)):
            return f"{label}: reconstruction differs in rows [{a}, {b})"
        return None

    errs = [e for e in _pool_map(one, _chunks(R, max(1, (1 << 21) // d))) if e]
    assert not errs, errs[0]


def residual_every_row(k: np.ndarray, S: np.ndarray, g: int, codes: np.ndarray,
                       steps: np.ndarray, offsets: np.ndarray, words: np.ndarray,
                       norms: np.ndarray) -> tuple[int, int]:
    """Two-stage compression of every row of k [R, d]: the INT4 part bit for
    bit (offsets by value), the residual's sign bits within the 1e-4
    ||S_i|| ||r|| band and its norm within one binary16 ulp.  Returns
    (differing bits, norms off by one ulp)."""
    from oracle import int4 as O4, residual as OR
    R, d = k.shape
    m = S.shape[0]
    words = words.reshape(R, m // 32)
    s_norm = np.linalg.norm(S.astype(np.float64), axis=1)

    def one(span):
        a, b = span
        co, so, zo = O4.quantize_int4(k[a:b], g)
        if not np.array_equal(codes[a:b], co):
            return f"INT4 codes differ in rows [{a}, {b})", 0, 0
        if not np.array_equal(steps[a:b].view(np.uint32), so.view(np.uint32)):
            return f"INT4 steps differ in rows [{a}, {b})", 0, 0
        if not np.array_equal(offsets[a:b], zo):
            return f"INT4 offsets differ in rows [{a}, {b})", 0, 0
        r = OR.residual(k[a:b], O4.dequantize_int4(co, so, zo, g))
        P = OQ.project(r, S)
        wo = OQ.pack_signs(P >= 0.0)
        flips = 0
        bad = np.nonzero((words[a:b] != wo).any(axis=1))[0]
        if len(bad):
            diff = OQ.unpack_signs(words[a:b][bad], m) != OQ.unpack_signs(wo[bad], m)
            rn = np.linalg.norm(r[bad].astype(np.float64), axis=1)
            if (diff & (np.abs(P[bad]) > 1e-4 * rn[:, None] * s_norm[None, :])).any():
                return f"residual sign bits differ outside the band in rows [{a}, {b})", 0, 0
            flips = int(diff.sum())
        no = OQ.key_norms(r).view(np.uint16).astype(np.int64)
        ng = norms[a:b].view(np.uint16).astype(np.int64)
        if np.any(np.abs(no - ng) > 1):
            return f"residual norms differ by more than one ulp in rows [{a}, {b})", 0, 0
        return None, flips, int((no != ng).sum())

    res = _pool_map(one, _chunks(R, 1 << 15))
    errs = [e for e, _, _ in res if e]
    assert not errs, errs[0]
    return sum(f for _, f, _ in res), sum(n for _, _, n in res)


def int8_scores_every_score(q: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                            scores: np.ndarray) -> float:
    """|gpu - ora| <= 1e-5 s_t sum_i |q_i c_ti| for every score of q [G, nq, d]
    against codes [G, T, d], scales [G, T]; returns the worst err / scale."""
    G, T, d = codes.shape

    def one(span):
        g, a, b = span
        ora = OI.scores_int8(q[g:g + 1], codes[g:g + 1, a:b], scales[g:g + 1, a:b])
        mag = np.matmul(np.abs(q[g:g + 1].astype(np.float64)),
                        np.swapaxes(np.abs(codes[g:g + 1, a:b].astype(np.float64)), 1, 2))
        mag *= scales[g:g + 1, a:b].astype(np.float64)[:, None, :]
        err = np.abs(scores[g:g + 1, :, a:b].astype(np.float64) - ora)
        if np.any(err > 1e-5 * mag + 1e-30):
            return f"INT8 scores of group {g}, tokens [{a}, {b}) outside 1e-5", 0.0
        return None, float(np.max(err / (mag + 1e-30)))

    spans = [(g, a, b) for g in range(G) for a, b in _chunks(T, 1 << 16)]
    res = _pool_map(one, spans)
    errs = [e for e, _ in res if e]
    assert not errs, errs[0]
    return max(w for _, w in res)
