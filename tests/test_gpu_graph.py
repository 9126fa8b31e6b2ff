"""The decode step (compress the newest token into the cache, then decode)
captured in a HIP graph gives, on every replay, exactly the output of the
same calls made eagerly: the library's launches make no allocation and no
memset, so they are safe to capture.  Replays are interleaved with eager
work and new inputs written into the captured tensors between them."""
import math

import numpy as np
import pytest
import torch

import kv_cache_compression_kvq_amd as K
from gpu_common import log

pytestmark = pytest.mark.gpu


def make_state(seed, G, T, d, m):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    k = torch.randn(G, T, d, device="cuda", generator=g).half()
    v = torch.randn(G, T, d, device="cuda", generator=g).half()
    S = torch.randn(m, d, device="cuda", generator=g).half()
    kbits, knorms = K.qjl_sketch(k, S)
    vcodes, vscales = K.quantize_int8(v)
    q = torch.randn(G, d, device="cuda", generator=g).half()
    k_new = torch.randn(G, d, device="cuda", generator=g).half()
    v_new = torch.randn(G, d, device="cuda", generator=g).half()
    return dict(S=S, kbits=kbits, knorms=knorms, vcodes=vcodes, vscales=vscales, q=q,
                k_new=k_new, v_new=v_new)


def step(st, ws, out, T):
    """Newest token into position T - 1 (the fused append), then decode; the
    standalone quantizer and sketch of the same token go to position T - 2."""
    K.cache_append(st["k_new"], st["v_new"], st["S"], st["kbits"], st["knorms"], st["vcodes"],
                   st["vscales"], T - 1)
    vc, vs = K.quantize_int8(st["v_new"])
    kb, kn = K.qjl_sketch(st["k_new"], st["S"])
    st["vcodes"][:, T - 2].copy_(vc)
    st["vscales"][:, T - 2].copy_(vs)
    st["kbits"][:, T - 2].copy_(kb)
    st["knorms"][:, T - 2].copy_(kn)
    K.decode_qjl_int8(st["q"], st["S"], st["kbits"], st["knorms"], st["vcodes"], st["vscales"],
                      1 / math.sqrt(st["q"].shape[1]), workspace=ws, out=out)


def clone_state(st):
    return {k: v.clone() for k, v in st.items()}


@pytest.mark.parametrize("G,T,d,m", [(8, 3000, 128, 256), (5, 777, 64, 128)])
def test_graph_replays_match_eager(G, T, d, m):
    log(f"[graph] G={G} T={T} d={d} m={m}")
    st = make_state(11 + d, G, T, d, m)
    ws = torch.empty(max(16, K.decode_workspace_bytes(G, T, d, m)), dtype=torch.uint8, device="cuda")
    out = torch.empty(G, d, dtype=torch.float32, device="cuda")
    st_eager = clone_state(st)
    ws_e = torch.empty_like(ws)
    out_e = torch.empty_like(out)

    step(st, ws, out, T)                  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(st, ws, out, T)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for rep in range(4):
        if rep:                           # new query and newest token for this replay
            for key in ("q", "k_new", "v_new"):
                st[key].copy_(torch.randn(st[key].shape, device="cuda", generator=gen).half())
                st_eager[key].copy_(st[key])
        graph.replay()
        torch.cuda.synchronize()
        # eager work between replays, on the same stream
        _ = K.scores_qjl(st_eager["q"][:, None, :], st_eager["S"], st_eager["kbits"],
                         st_eager["knorms"])
        step(st_eager, ws_e, out_e, T)
        torch.cuda.synchronize()
        a, b = out.cpu().numpy(), out_e.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
            f"replay {rep}: max diff {np.max(np.abs(a - b))}"
        for key in ("kbits", "knorms", "vcodes", "vscales"):
            assert torch.equal(st[key], st_eager[key]), f"replay {rep}: cache {key} differs"
    log(f"[graph] 4 replays equal the eager step")
