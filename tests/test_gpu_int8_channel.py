"""GPU parity of per-channel INT8 keys against the oracle: codes, scales and
dequantised values bit-exact; scores within 1e-5 * sum_c |q_c s_c c_tc|.
Every call goes through the C ABI (libkvq.so)."""
import numpy as np
import pytest
import torch

import kv_cache_compression_kvq_amd as K
import synth_inputs as si
from oracle import int8_channel as OC
from gpu_common import down, log, up

pytestmark = pytest.mark.gpu


def roundtrip_check(x: np.ndarray, label: str):
    log(f"[int8ch] {label}: x {x.shape} {x.dtype}")
    cg_t, sg_t = K.quantize_int8_channel(up(x))
    co, so = OC.quantize_int8_channel(x)
    cg, sg = down(cg_t), down(sg_t)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32)), f"{label}: scales differ"
    if not np.array_equal(cg, co):
        g, t, c = np.nonzero(cg != co)
        raise AssertionError(f"{label}: {len(g)} codes differ, first at ({g[0]}, {t[0]}, {c[0]}): "
                             f"x={x[g[0], t[0], c[0]]!r} gpu={cg[g[0], t[0], c[0]]} "
                             f"oracle={co[g[0], t[0], c[0]]}")
    for out_dt, name, u in ((torch.float32, "f32", np.uint32), (torch.float16, "f16", np.uint16)):
        dg = down(K.dequantize_int8_channel(cg_t, sg_t, out_dt))
        do = OC.dequantize_int8_channel(co, so, name)
        assert np.array_equal(dg.view(u), do.view(u)), f"{label}: {name} reconstruction differs"
    return co, so


def scores_check(q, codes, scales, label):
    sc = down(K.scores_int8_channel(up(q), up(codes), up(scales)))
    ora = OC.scores_int8_channel(q, codes, scales)
    qs = np.abs(q.astype(np.float64) * scales.astype(np.float64)[:, None, :])
    tol = 1e-5 * np.matmul(qs, np.abs(np.swapaxes(codes.astype(np.float64), 1, 2)))
    err = np.abs(sc.astype(np.float64) - ora)
    bad = err > tol + 1e-30
    assert not bad.any(), f"{label}: {bad.sum()} scores outside the tolerance"
    log(f"[int8ch] {label}: worst err / tol = {np.max(err / (tol + 1e-30)):.3g}")


def test_llama_layer_keys_full_size():
    """Llama-7B-shaped keys: 32 heads x 4096 tokens x 128, fp16, with fixed
    outlier channels (where one scale per channel pays off)."""
    W = si.W_LLAMA_LAYER
    k = si.kv_tensor(W, si.K, 1, 32, 4096, 128, "f16", outliers=True).reshape(32, 4096, 128)
    codes, scales = roundtrip_check(k, "llama K")
    q = si.queries(W, 32, 1, 128, "f16")
    scores_check(q, codes, scales, "llama scores")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("d", [16, 48, 128, 1024, 2048, 8192])
def test_shapes_and_ragged_token_counts(dtype, d):
    rng = np.random.default_rng(d)
    for T in (1, 3, 127, 128, 129, 255, 256, 257, 1000) if d <= 1024 else (1, 129, 300):
        G = 3
        x = rng.standard_normal((G, T, d)).astype(np.float32)
        x *= np.exp(rng.uniform(-6, 6, (G, 1, d))).astype(np.float32)
        if dtype == "f16":
            x = np.clip(x, -6e4, 6e4).astype(np.float16)
        roundtrip_check(x, f"{dtype} d={d} T={T}")


@pytest.mark.parametrize("dtype", ["f32", "f16"])
@pytest.mark.parametrize("G", [8, 9])
def test_one_launch_token_limits(dtype, G):
    """Token counts around the one-launch kernel's register schedule (256
    tokens per load step, 2 to 16 steps, at most 4096 tokens) and just past
    it, where the slab passes take over; G = 8 places a group's workgroups
    on one XCD, G = 9 does not."""
    rng = np.random.default_rng(G * 7 + len(dtype))
    for T in (2, 512, 513, 1024, 1025, 2048, 2049, 4095, 4096, 4097):
        d = 128 if T > 1024 else 48
        x = rng.standard_normal((G, T, d)).astype(np.float32)
        x *= np.exp(rng.uniform(-4, 4, (G, 1, d))).astype(np.float32)
        x[:, rng.integers(0, T), :] *= 50.0            # one loud token per group
        if dtype == "f16":
            x = np.clip(x, -6e4, 6e4).astype(np.float16)
        roundtrip_check(x, f"{dtype} G={G} T={T} d={d}")


def test_many_slabs():
    """T = 5000 (40 slabs of 128 tokens) for 5 groups, fp32 and fp16."""
    rng = np.random.default_rng(50)
    x = (rng.standard_normal((5, 5000, 64)) * rng.uniform(0.1, 50, (5, 1, 64))).astype(np.float32)
    roundtrip_check(x, "fp32 T=5000")
    roundtrip_check(x.astype(np.float16), "fp16 T=5000")


@pytest.mark.parametrize("dtype", [np.float32, np.float16])
def test_special_channels(dtype):
    T, d = 300, 32
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, T, d))
    x[0, :, 0] = 0                                     # all-zero channel
    x[0, :, 1] = -0.0
    x[0, :, 2] = 0
    x[0, 17, 2] = 1e4 if dtype == np.float16 else 1e30   # one spike
    x[0, :, 3] = (np.arange(T) % 255 - 127) + 0.5      # half-integer quotients (s = 1 after max 127)
    x[0, 0, 3] = 127
    x[1, :, 4] = 0.25                                  # constant channel
    if dtype == np.float32:
        x[1, :, 5] = 0
        x[1, 3, 5] = 2.0 ** -149                       # scale underflows to 0
        x[1, :, 6] = np.linspace(-1e-38, 1e-38, T)     # subnormal values
    roundtrip_check(x.astype(dtype), f"special channels {np.dtype(dtype).name}")


@pytest.mark.parametrize("qdt", ["f16", "f32"])
@pytest.mark.parametrize("nq,T,d", [(1, 1, 128), (4, 300, 128), (1, 2049, 64), (8, 77, 1024),
                                    (2, 1000, 48), (1, 33, 8192)])
def test_scores_shapes(qdt, nq, T, d):
    rng = np.random.default_rng(nq * 31 + T)
    G = 3
    x = (rng.standard_normal((G, T, d)) * rng.uniform(0.1, 20, (G, 1, d))).astype(np.float32)
    codes, scales = OC.quantize_int8_channel(x)
    q = rng.standard_normal((G, nq, d)).astype(np.float16 if qdt == "f16" else np.float32)
    scores_check(q, codes, scales, f"{qdt} nq={nq} T={T} d={d}")


@pytest.mark.parametrize("qdt", ["f16", "f32"])
@pytest.mark.parametrize("nq", [2, 4, 8])
def test_scores_grouped_queries_matrix_cores(qdt, nq):
    """d = 128, 2 .. 8 queries per group: the matrix-core score with the
    per-channel products q_c s_c split hi / lo, channel scales spanning
    many binades."""
    rng = np.random.default_rng(nq * 5 + len(qdt))
    for G, T in ((2, 3), (3, 300), (2, 5000)):
        x = (rng.standard_normal((G, T, 128)) * np.exp(rng.uniform(-8, 8, (G, 1, 128)))).astype(np.float32)
        codes, scales = OC.quantize_int8_channel(x)
        q = rng.standard_normal((G, nq, 128)).astype(np.float16 if qdt == "f16" else np.float32)
        scores_check(q, codes, scales, f"{qdt} nq={nq} T={T} d=128")


def test_empty_inputs_are_noops():
    x = torch.empty((2, 0, 128), dtype=torch.float16, device="cuda")
    codes, scales = K.quantize_int8_channel(x)
    assert codes.shape == (2, 0, 128) and scales.shape == (2, 128)
    q = torch.zeros((2, 1, 128), dtype=torch.float16, device="cuda")
    out = K.scores_int8_channel(q, codes, torch.zeros((2, 128), dtype=torch.float32, device="cuda"))
    assert out.shape == (2, 1, 0)
