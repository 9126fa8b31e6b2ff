"""GPU parity of kvq_cache_append (compress-on-write of the newest token of
every group into cache position pos) against the oracle: value codes and
scales bit-exact, sign bits equal outside the 1e-4 band, norms within one
binary16 ulp, and every other cache row left as it was."""
import numpy as np
import pytest
import torch

import kv_cache_compression_kvq_amd as K
from oracle import int8 as OI, qjl as OQ
from gpu_common import assert_bits_within_band, assert_norms_within_ulp, down, log, up

pytestmark = pytest.mark.gpu


def random_cache(rng, G, T, d, m):
    """Arbitrary bytes in every cache tensor (the append must not read them)."""
    kb = rng.integers(0, 2 ** 32, (G, T, m // 32), dtype=np.uint32)
    kn = rng.standard_normal((G, T)).astype(np.float16)
    vc = rng.integers(-128, 128, (G, T, d), dtype=np.int8)
    vs = rng.random((G, T)).astype(np.float32)
    return kb, kn, vc, vs


@pytest.mark.parametrize("G,T,d,m,dt,pos", [
    (13, 50, 128, 256, "f16", 49),     # ragged last workgroup (13 = 8 + 5)
    (8, 1, 64, 32, "f32", 0),          # T = 1, smallest m
    (3, 7, 1024, 1024, "f16", 3),      # largest d and m
    (1, 5, 16, 64, "f32", 2),          # smallest d
    (512, 4, 128, 256, "f16", 3),      # the decode workload's group count
    (9, 3, 96, 160, "f32", 1),         # m not a multiple of 64
])
def test_append_matches_oracle(G, T, d, m, dt, pos):
    log(f"[append] G={G} T={T} d={d} m={m} {dt} pos={pos}")
    rng = np.random.default_rng(G * 1000 + d + m)
    npdt = np.float16 if dt == "f16" else np.float32
    k = rng.standard_normal((G, d)).astype(npdt)
    v = (rng.standard_normal((G, d)) * rng.choice([1e-3, 1.0, 50.0], (G, 1))).astype(npdt)
    v[0, :] = 0                                             # an all-zero value row
    S = rng.standard_normal((m, d)).astype(npdt)
    kb, kn, vc, vs = random_cache(rng, G, T, d, m)
    tk, tn, tc, ts = up(kb), up(kn), up(vc), up(vs)
    K.cache_append(up(k), up(v), up(S), tk, tn, tc, ts, pos)
    gk, gn = down(tk, np.uint32), down(tn)
    gc, gs = down(tc), down(ts)

    rest = np.ones(T, bool)
    rest[pos] = False
    assert np.array_equal(gk[:, rest], kb[:, rest])
    assert np.array_equal(gn[:, rest].view(np.uint16), kn[:, rest].view(np.uint16))
    assert np.array_equal(gc[:, rest], vc[:, rest])
    assert np.array_equal(gs[:, rest].view(np.uint32), vs[:, rest].view(np.uint32))

    ocodes, oscales = OI.quantize_int8(v)
    assert np.array_equal(gc[:, pos], ocodes)
    assert np.array_equal(gs[:, pos].view(np.uint32), oscales.view(np.uint32))
    owords, onorms = OQ.qjl_sketch(k, S)
    nflip = assert_bits_within_band(gk[:, pos], owords, k, S)
    assert_norms_within_ulp(gn[:, pos], onorms)
    log(f"[append] ok ({nflip} sign bits inside the band)")


def test_append_equals_standalone_kernels():
    """Codes, scales and norms of the append equal kvq_quantize_int8 and the
    oracle norms; at the decode workload's shape the bits agree with
    kvq_qjl_sketch except inside the band."""
    rng = np.random.default_rng(4)
    G, T, d, m = 512, 3, 128, 256
    k = rng.standard_normal((G, d)).astype(np.float16)
    v = rng.standard_normal((G, d)).astype(np.float16)
    S = rng.standard_normal((m, d)).astype(np.float16)
    kb, kn, vc, vs = random_cache(rng, G, T, d, m)
    tk, tn, tc, ts = up(kb), up(kn), up(vc), up(vs)
    K.cache_append(up(k), up(v), up(S), tk, tn, tc, ts, T - 1)
    c2, s2 = K.quantize_int8(up(v))
    b2, n2 = K.qjl_sketch(up(k), up(S))
    assert torch.equal(tc[:, T - 1], c2)
    assert torch.equal(ts[:, T - 1], s2)
    assert_bits_within_band(down(tk[:, T - 1], np.uint32), down(b2, np.uint32), k, S)
    assert_norms_within_ulp(down(tn[:, T - 1]), down(n2))


def test_append_no_groups_is_a_noop():
    z = torch.empty(0, 128, dtype=torch.float16, device="cuda")
    S = torch.zeros(256, 128, dtype=torch.float16, device="cuda")
    kb = torch.empty(0, 4, 8, dtype=torch.int32, device="cuda")
    kn = torch.empty(0, 4, dtype=torch.float16, device="cuda")
    vc = torch.empty(0, 4, 128, dtype=torch.int8, device="cuda")
    vs = torch.empty(0, 4, dtype=torch.float32, device="cuda")
    K.cache_append(z, z, S, kb, kn, vc, vs, 0)
