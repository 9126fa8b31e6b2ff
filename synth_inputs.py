"""Seeded synthetic inputs shared by the oracle, the GPU tests and the bench.

This module only draws random numbers and lays them out; it holds none of
the compression arithmetic.  Every tensor is a deterministic function of
(workload id, tensor id, element range), so any slice (one head, one group,
a sampled row) can be regenerated on its own without materialising the rest.

Recipe
------
* Element stream of tensor ``t`` in workload ``w``: chunk ``j`` (2**24
  elements) is ``np.random.default_rng([0, w, t, j]).standard_normal(n,
  dtype=float32)``; the stream is cut into rows in row-major order.
* fp16 tensors are drawn in fp32 and rounded to fp16 (round-to-nearest-even).
* Key outliers: per head, 4 distinct channels are drawn once from
  ``default_rng([0, w, 5, head]).choice(d, 4, replace=False)``; those
  channels are multiplied by 20 in fp32 before the fp16 rounding, for every
  token and batch entry of that head.
* The JL matrix S ``[m, d]`` is ``default_rng([0, w, 4]).standard_normal((m, d))``
  in float64, rounded to the key dtype.
* ``uniform`` streams (the U(-1, 1) context row) use ``rng.random`` in fp32
  mapped to [-1, 1).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 24
ROOT_SEED = 0

# tensor ids inside a workload
K, V, Q, S_ID, OUTLIER = 1, 2, 3, 4, 5

# workload ids: the five named workloads, then small test-only shapes
W_TINY, W_LLAMA_LAYER, W_SWEEP, W_QJL_CACHE, W_DECODE = 1, 2, 3, 4, 5

_NP_DTYPES = {"f32": np.float32, "f16": np.float16}


def _chunk(w: int, t: int, j: int, n: int, dist: str) -> np.ndarray:
    rng = np.random.default_rng([ROOT_SEED, w, t, j])
    if dist == "normal":
        return rng.standard_normal(n, dtype=np.float32)
    if dist == "uniform":
        return rng.random(n, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    raise ValueError(dist)


def stream(w: int, t: int, n: int, dtype: str = "f32", start: int = 0,
           dist: str = "normal", workers: int | None = None) -> np.ndarray:
    """Elements [start, start+n) of tensor t of workload w, as a flat array.

    Chunk j of the stream is the first 2**24 draws of its own generator; a
    request that needs only a prefix of a chunk draws only that prefix (the
    generator fills sequentially, so a prefix equals the same slice of the
    full chunk).  Chunks are independent, so large requests are filled by a
    thread pool (numpy's generators release the GIL); the bytes do not
    depend on the number of workers.
    """
    np_dt = _NP_DTYPES[dtype]
    out = np.empty(n, dtype=np_dt)
    stop = start + n
    pieces = []
    pos = start
    while pos < stop:
        j = pos // CHUNK
        take = min(stop, (j + 1) * CHUNK) - pos
        pieces.append((j, pos - j * CHUNK, take))
        pos += take

    def fill(piece):
        j, lo, take = piece
        c = _chunk(w, t, j, lo + take, dist)
        dst = j * CHUNK + lo - start
        out[dst: dst + take] = c[lo:].astype(np_dt)

    nworkers = workers or min(16, len(os.sched_getaffinity(0)))
    if len(pieces) > 1 and nworkers > 1:
        with ThreadPoolExecutor(max_workers=nworkers) as ex:
            list(ex.map(fill, pieces))
    else:
        for pc in pieces:
            fill(pc)
    return out


def outlier_channels(w: int, n_heads: int, d: int, count: int = 4) -> np.ndarray:
    """[n_heads, count] distinct channel indices per head."""
    out = np.empty((n_heads, count), dtype=np.int64)
    for h in range(n_heads):
        out[h] = np.random.default_rng([ROOT_SEED, w, OUTLIER, h]).choice(d, count, replace=False)
    return out


def kv_tensor(w: int, t: int, B: int, H: int, T: int, d: int, dtype: str,
              outliers: bool = False, heads: range | None = None,
              tokens: range | None = None, dist: str = "normal") -> np.ndarray:
    """A [B, H, T, d] K or V tensor (or a head/token sub-block of it).

    ``heads`` / ``tokens`` select a sub-block of every batch entry without
    generating the rest; the values equal the same slice of the full tensor.
    """
    heads = heads if heads is not None else range(H)
    tokens = tokens if tokens is not None else range(T)
    full = (len(heads) == H and len(tokens) == T)
    if full:
        x = stream(w, t, B * H * T * d, "f32", dist=dist).reshape(B, H, T, d)
    else:
        x = np.empty((B, len(heads), len(tokens), d), dtype=np.float32)
        for b in range(B):
            for hi, h in enumerate(heads):
                base = ((b * H + h) * T + tokens.start) * d
                x[b, hi] = stream(w, t, len(tokens) * d, "f32", start=base, dist=dist).reshape(len(tokens), d)
    if outliers:
        ch = outlier_channels(w, H, d)
        for hi, h in enumerate(heads):
            x[:, hi, :, ch[h]] *= np.float32(20.0)
    return x.astype(_NP_DTYPES[dtype]) if dtype != "f32" else x


def projection(w: int, m: int, d: int, dtype: str) -> np.ndarray:
    """The JL matrix S [m, d] with N(0, 1) entries, rounded to ``dtype``."""
    s = np.random.default_rng([ROOT_SEED, w, S_ID]).standard_normal((m, d))
    return s.astype(_NP_DTYPES[dtype])


def queries(w: int, G: int, nq: int, d: int, dtype: str) -> np.ndarray:
    """Decode queries [G, nq, d] ~ N(0, 1)."""
    return stream(w, Q, G * nq * d, dtype).reshape(G, nq, d)


def flat_rows(w: int, n_elems: int, d: int, dtype: str = "f32",
              dist: str = "normal", rows: range | None = None) -> np.ndarray:
    """A flat tensor of n_elems elements viewed as [n_elems // d, d] rows
    (tensor id K); ``rows`` selects a row range of it."""
    if rows is None:
        return stream(w, K, n_elems, dtype, dist=dist).reshape(-1, d)
    return stream(w, K, (rows.stop - rows.start) * d, dtype, start=rows.start * d,
                  dist=dist).reshape(-1, d)
