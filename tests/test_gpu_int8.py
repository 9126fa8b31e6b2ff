"""GPU parity of the INT8 path against the oracle: codes, scales and
dequantised values bit-exact; scale-folded scores within
1e-5 * s * sum|q c|.  Every call goes through the C ABI (libkvq.so)."""
import numpy as np
import pytest
import torch

import kv_cache_compression_kvq_amd as K
import synth_inputs as si
from oracle import int8 as O
import full_size as FS
from gpu_common import assert_int8_scores, down, log, up

pytestmark = pytest.mark.gpu


def roundtrip_check(x: np.ndarray, label: str):
    """Quantize + dequantize x [R, d] on the GPU; compare bit-exactly."""
    log(f"[int8] {label}: x {x.shape} {x.dtype}")
    codes_g, scales_g = K.quantize_int8(up(x))
    codes_o, scales_o = O.quantize_int8(x)
    cg, sg = down(codes_g), down(scales_g)
    assert np.array_equal(sg.view(np.uint32), scales_o.view(np.uint32)), f"{label}: scales differ"
    if not np.array_equal(cg, codes_o):
        r, c = np.nonzero(cg != codes_o)
        raise AssertionError(f"{label}: {len(r)} codes differ, first at row {r[0]} col {c[0]}: "
                             f"x={x[r[0], c[0]]!r} gpu={cg[r[0], c[0]]} oracle={codes_o[r[0], c[0]]}")
    out_dt = torch.float16 if x.dtype == np.float16 else torch.float32
    deq_g = down(K.dequantize_int8(codes_g, scales_g, out_dt))
    deq_o = O.dequantize_int8(codes_o, scales_o, "f16" if x.dtype == np.float16 else "f32")
    u = np.uint16 if x.dtype == np.float16 else np.uint32
    assert np.array_equal(deq_g.view(u), deq_o.view(u)), f"{label}: dequantised values differ"
    return codes_o, scales_o


# --- tiny workload: one layer, one head, 512 tokens, d = 128, fp32 -----------

def test_tiny_layer_kv_and_scores():
    W = si.W_TINY
    k = si.kv_tensor(W, si.K, 1, 1, 512, 128, "f32")
    v = si.kv_tensor(W, si.V, 1, 1, 512, 128, "f32")
    kc, ks = roundtrip_check(k.reshape(-1, 128), "tiny K")
    roundtrip_check(v.reshape(-1, 128), "tiny V")
    q = si.queries(W, 1, 4, 128, "f32")
    sc = down(K.scores_int8(up(q), up(kc.reshape(1, 512, 128)), up(ks.reshape(1, 512))))
    ora = O.scores_int8(q, kc.reshape(1, 512, 128), ks.reshape(1, 512))
    worst = assert_int8_scores(sc, q, kc.reshape(1, 512, 128), ks.reshape(1, 512), ora)
    log(f"[int8] tiny scores: worst err / tol-scale = {worst:.3g}")


# --- Llama-7B-shaped layer: 32 heads x 4096 tokens x 128, fp16, outliers --------

def test_llama_layer_full_size():
    W = si.W_LLAMA_LAYER
    k = si.kv_tensor(W, si.K, 1, 32, 4096, 128, "f16", outliers=True)
    v = si.kv_tensor(W, si.V, 1, 32, 4096, 128, "f16")
    kc, ks = roundtrip_check(k.reshape(-1, 128), "llama K")
    roundtrip_check(v.reshape(-1, 128), "llama V")
    q = si.queries(W, 32, 1, 128, "f16")
    codes = kc.reshape(32, 4096, 128)
    scales = ks.reshape(32, 4096)
    sc = down(K.scores_int8(up(q), up(codes), up(scales)))
    ora = O.scores_int8(q, codes, scales)
    worst = assert_int8_scores(sc, q, codes, scales, ora)
    log(f"[int8] llama scores: worst err / tol-scale = {worst:.3g}")


# --- element-count sweep ---------------------------------------------------------

@pytest.mark.parametrize("n_log2", [20, 24])
@pytest.mark.parametrize("d", [128, 1024, 8192])
def test_sweep_small_sizes_full_compare(n_log2, d):
    x = si.flat_rows(si.W_SWEEP, 1 << n_log2, d)
    roundtrip_check(x, f"sweep 2^{n_log2} d={d}")


@pytest.mark.parametrize("n_log2", [28, 30])
def test_sweep_large_sizes_every_row(n_log2):
    """2^28 and 2^30 fp32 elements as rows of 128, 1024 and 8192 (the bench's
    launches): every row is quantized and dequantized on the GPU and every
    code, scale and dequantised value is compared bit-exactly with the
    oracle's (chunked over a thread pool on the host)."""
    n = 1 << n_log2
    x_host = si.flat_rows(si.W_SWEEP, n, 128).reshape(-1)   # same bytes for every d
    x = up(x_host)
    for d in (128, 1024, 8192):
        rows = n // d
        xv = x.view(rows, d)
        log(f"[int8] sweep 2^{n_log2} d={d}: quantize {rows} rows")
        codes, scales = K.quantize_int8(xv)
        deq = K.dequantize_int8(codes, scales)
        c, s, dq = down(codes), down(scales), down(deq)
        del codes, scales, deq
        FS.int8_every_row(x_host.reshape(rows, d), c, s, dq, f"sweep 2^{n_log2} d={d}")
        err = np.abs(x_host.reshape(rows, d) - dq)
        log(f"[int8] sweep 2^{n_log2} d={d}: every row bit-exact; max|x-x_hat| {float(err.max()):.4g}")
        del c, s, dq, err
    # the host copy is the generator's stream: spot-check one row
    row = si.flat_rows(si.W_SWEEP, n, 128, rows=range(12345, 12346))
    assert np.array_equal(x_host.reshape(-1, 128)[12345:12346], row)


# --- edge cases -------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("d", [16, 32, 48, 64, 80, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 1040])
def test_shapes_and_ragged_rows(dtype, d):
    rng = np.random.default_rng(d)
    for rows in (1, 3, 63, 129, 1000):
        x = rng.standard_normal((rows, d)).astype(np.float32)
        x *= np.exp(rng.uniform(-8, 8, (rows, 1))).astype(np.float32)
        if dtype == "f16":
            x = x.astype(np.float16)
        roundtrip_check(x, f"{dtype} d={d} rows={rows}")


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_special_rows(dtype):
    d = 128
    rows = []
    rows.append(np.zeros(d))                                  # zero row
    rows.append(-np.zeros(d))                                 # negative zeros
    rows.append(np.full(d, 0.3))                              # all equal
    rows.append(np.full(d, -7.25))
    z = np.zeros(d); z[17] = 1e4 if dtype == np.float16 else 1e30; rows.append(z)   # one spike
    rows.append(np.arange(d) - 63.5)                          # ties on the half-integers
    rows.append((np.arange(d) - 64) * 0.5)                    # many x.5 quotients
    if dtype == np.float32:
        z = np.zeros(d); z[0] = 2.0 ** -149; rows.append(z)   # scale underflows to 0
        z = np.zeros(d); z[0] = 2.0 ** -135; z[1] = -2.0 ** -136; rows.append(z)  # subnormal scale
        rows.append(np.linspace(-1e-38, 1e-38, d))            # subnormal inputs
    else:
        z = np.zeros(d); z[0] = 2.0 ** -24; rows.append(z)    # smallest fp16 subnormal
    x = np.array(rows).astype(dtype)
    roundtrip_check(x, f"special rows {np.dtype(dtype).name}")


def test_near_tie_quotients():
    """Rows where x / s lands within a few ulps of half-integers."""
    rng = np.random.default_rng(77)
    R, d = 4096, 128
    a = (np.abs(rng.standard_normal(R)) * 10.0 ** rng.integers(-5, 6, R) + 1e-6).astype(np.float32)
    s = (a.astype(np.float64) / 127.0).astype(np.float32)
    k = rng.integers(-127, 127, (R, d)) + 0.5
    base = (k * s.astype(np.float64)[:, None]).astype(np.float32)
    steps = rng.integers(-2, 3, (R, d)).astype(np.int32)
    x = (base.view(np.int32) + steps * np.sign(base).astype(np.int32)).view(np.float32)
    x = np.clip(x, -a[:, None], a[:, None])
    x[:, 0] = a
    roundtrip_check(x.astype(np.float32), "near ties")


def test_exhaustive_fp16_values():
    """Every finite binary16 value, in rows whose max is 65504 or 1.0."""
    allf = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    allf = allf[np.isfinite(allf)]
    pad = (-len(allf)) % 127
    vals = np.concatenate([allf, np.zeros(pad, np.float16)]).reshape(-1, 127)
    big = np.concatenate([np.full((vals.shape[0], 1), 65504, np.float16), vals], axis=1)
    roundtrip_check(big, "all fp16 values, max 65504")
    small = np.where(np.abs(vals.astype(np.float32)) <= 1.0, vals, np.float16(0.5))
    small = np.concatenate([np.ones((vals.shape[0], 1), np.float16), small], axis=1)
    roundtrip_check(small, "all fp16 values <= 1, max 1")


@pytest.mark.parametrize("qdt", ["f32", "f16"])
@pytest.mark.parametrize("nq,T,d", [(1, 1, 128), (3, 77, 128), (5, 300, 64), (8, 129, 256),
                                    (2, 1000, 48), (64, 33, 128), (1, 17, 16384)])
def test_scores_shapes(qdt, nq, T, d):
    rng = np.random.default_rng(nq * 1000 + T)
    G = 3
    x = rng.standard_normal((G * T, d)).astype(np.float32)
    codes, scales = O.quantize_int8(x)
    codes, scales = codes.reshape(G, T, d), scales.reshape(G, T)
    q = rng.standard_normal((G, nq, d)).astype(np.float16 if qdt == "f16" else np.float32)
    sc = down(K.scores_int8(up(q), up(codes), up(scales)))
    assert_int8_scores(sc, q, codes, scales, O.scores_int8(q, codes, scales))


@pytest.mark.parametrize("qdt", ["f32", "f16"])
@pytest.mark.parametrize("nq", [2, 3, 5, 8, 9, 16])
def test_scores_grouped_queries_matrix_cores(qdt, nq):
    """d = 128 with 2 .. 16 queries per group (the matrix-core score: fp16
    queries as 16 columns, fp32 queries split hi / lo into 8 + 8 columns,
    so fp32 with 9 and 16 queries takes the vector-ALU kernel; 2 and 3
    queries take it too below 2^20 rows), ragged token counts on both
    sides of the 256- and 1024-token block steps."""
    rng = np.random.default_rng(nq * 17 + len(qdt))
    for G, T in ((3, 1), (2, 17), (3, 255), (2, 1025), (5, 4099)):
        x = rng.standard_normal((G * T, 128)).astype(np.float32)
        x *= np.exp(rng.uniform(-3, 3, (G * T, 1))).astype(np.float32)
        codes, scales = O.quantize_int8(x)
        codes, scales = codes.reshape(G, T, 128), scales.reshape(G, T)
        q = rng.standard_normal((G, nq, 128)) * np.exp(rng.uniform(-4, 4, (G, nq, 1)))
        q = q.astype(np.float16 if qdt == "f16" else np.float32)
        sc = down(K.scores_int8(up(q), up(codes), up(scales)))
        assert_int8_scores(sc, q, codes, scales, O.scores_int8(q, codes, scales))


@pytest.mark.parametrize("qdt", ["f32", "f16"])
@pytest.mark.parametrize("nq", [2, 3])
def test_scores_few_queries_large_cache_matrix_cores(qdt, nq):
    """2 and 3 queries per group over 2^20 rows or more (the matrix-core
    score; smaller caches take the vector-ALU kernel), ragged last tile:
    every score compared with the oracle."""
    G, T, d = 2, (1 << 19) + 77, 128
    rng = np.random.default_rng(60 + nq + len(qdt))
    codes = rng.integers(-127, 128, size=(G, T, d), dtype=np.int8)
    scales = rng.uniform(1e-3, 5e-2, size=(G, T)).astype(np.float32)
    q = rng.standard_normal((G, nq, d)).astype(np.float16 if qdt == "f16" else np.float32)
    log(f"[int8] large-cache scores nq={nq} {qdt}")
    sc = down(K.scores_int8(up(q), up(codes), up(scales)))
    worst = FS.int8_scores_every_score(q, codes, scales, sc)
    log(f"[int8] large-cache scores nq={nq} {qdt}: worst err / scale = {worst:.3g}")


@pytest.mark.parametrize("nq", [1, 4])
def test_scores_long_cache_every_score(nq):
    """32 heads x 262144 tokens x 128 (the bench's long-cache launch: 2 or 8
    token iterations per block): every score compared with the oracle."""
    G, T, d = 32, 262144, 128
    rng = np.random.default_rng(40 + nq)
    codes = rng.integers(-127, 128, size=(G, T, d), dtype=np.int8)
    scales = rng.uniform(1e-3, 5e-2, size=(G, T)).astype(np.float32)
    q = rng.standard_normal((G, nq, d)).astype(np.float16)
    log(f"[int8] long-cache scores nq={nq}")
    sc = down(K.scores_int8(up(q), up(codes), up(scales)))
    worst = FS.int8_scores_every_score(q, codes, scales, sc)
    log(f"[int8] long-cache scores nq={nq}: worst err / scale = {worst:.3g}")


@pytest.mark.parametrize("nq,G,T", [(1, 5, 60001), (4, 5, 60001), (4, 9, 131073)])
def test_scores_iteration_paths_ragged(nq, G, T):
    """Caches large enough for the 2- and 8-iteration blocks, with ragged
    last tiles: every score compared with the oracle."""
    rng = np.random.default_rng(nq * 7 + G)
    d = 128
    codes = rng.integers(-127, 128, size=(G, T, d), dtype=np.int8)
    scales = rng.uniform(1e-3, 5e-2, size=(G, T)).astype(np.float32)
    q = rng.standard_normal((G, nq, d)).astype(np.float32)
    sc = down(K.scores_int8(up(q), up(codes), up(scales)))
    assert_int8_scores(sc, q, codes, scales, O.scores_int8(q, codes, scales))


def test_empty_inputs_are_noops():
    x = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    c, s = K.quantize_int8(x)
    assert c.shape == (0, 128) and s.shape == (0,)
    q = torch.zeros((2, 1, 128), dtype=torch.float16, device="cuda")
    out = K.scores_int8(q, torch.empty((2, 0, 128), dtype=torch.int8, device="cuda"),
                        torch.empty((2, 0), dtype=torch.float32, device="cuda"))
    assert out.shape == (2, 1, 0)
