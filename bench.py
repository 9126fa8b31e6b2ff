"""Benchmark: one decode step over a compressed long-context KV cache on one
MI355X, plus the INT8 / QJL kernels on their own workloads.

Workload (one step): batch 16 x 32 heads x 32768 tokens x head dim 128.
The cache holds QJL-sketched keys (m = 256 sign bits + fp16 norm per token)
and per-token INT8 values (codes + fp32 scale), built once before timing
from fp16 N(0, 1) tensors.  A step
  1. compresses the newest token of every head: INT8-quantizes its value and
     QJL-sketches its key, written straight into cache position T - 1
     (kvq_cache_append, one launch);
  2. runs one decode query per head against all T tokens: QJL scores, fp32
     softmax and the weighted sum of INT8 values (kvq_decode_qjl_int8).
Steps are launched back to back and timed as a block (wall clock, with HIP
events at its two ends only).  Throughput is scores per second (query-token
pairs scored per step / time).

Also reported (``components``, sections copy / tiny / sweep / llama / qjl /
residual / gqa): the one-head fp32 correctness workload (launch-bound, for
context), HBM GB/s and roofline fractions of INT8 and INT4 quantize /
dequantize on the element-count sweep (2^28 and 2^30 fp32), the Llama-7B
layer (INT8, INT4, per-channel INT8, scores; also as HIP-graph replays), the
QJL-cache sketch and scores with their HBM stream references, the two-stage
compress and scores, and the grouped-query decode, each timed with HIP
events on the stream the kernels run on.  ``cpu_baseline`` times the fp64
oracle on bounded samples (the decode on one thread and on every thread,
the INT8 quantizer on the 2^28 sweep).

    python bench.py [--gpus 1] [--steps 50] [--warmup 1000] [--no-components]
                    [--config {all,tiny,llama7b,sweep,qjl,decode}]
                    [--only SECTIONS] [--no-cpu-baseline]

``--config`` picks one of the five workloads (the decode step alone, or
the component sections of one workload); the default runs all of them.

The default warm-up (1000 steps, ~0.45 s) brings the GPU's clocks up after
the seconds of host-side input generation before the timed region: with 3
warm-up steps the same 20 timed steps measured ~4 % slower.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_hbm_traffic.json")
DECODE_SOURCES = ["decode_kernels.hip", "kvq_qjl_device.h", "kvq_device.h"]


def parse_args():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=1000)
    p.add_argument("--no-components", action="store_true")
    p.add_argument("--only", default=",".join(SECTIONS),
                   help="comma-separated component sections to run (" + ", ".join(SECTIONS) + ")")
    p.add_argument("--config", default="all", choices=("all",) + tuple(CONFIGS),
                   help="one workload: tiny (1 head x 512 tokens x 128, fp32), llama7b (one "
                        "Llama-7B layer's K and V), sweep (2^28 and 2^30 fp32 elements), qjl "
                        "(8 x 32 x 8192 x 128 QJL key cache, grouped-query variants), decode "
                        "(the decode step only); all (default) runs every one")
    p.add_argument("--no-graph", action="store_true",
                   help="skip the HIP-graph replay timings (profiling aid)")
    p.add_argument("--no-decode", action="store_true",
                   help="skip the decode step (profiling aid: the line then has no value)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=6.0,
                   help="oracle compute time per CPU-baseline measurement (four of them)")
    p.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "CAL_FETCH_CSV",
                                                          "CAL_WRITE_CSV"),
                   help="CPU only: write the decode's HBM traffic per launch (profiles/"
                        "decode_split_hbm_traffic.json) from rocprofv3 --pmc FETCH_SIZE and "
                        "WRITE_SIZE counter_collection.csv files of a decode run and of a "
                        "--copy-calibration run")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a 1 GiB device-to-device copy 3 times (the known-size "
                        "kernel used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_source_hash() -> str:
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, "kv_cache_compression_kvq_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(bytes_per_launch_alg: float):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current decode sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except OSError:
        return None
    if t.get("source_sha") != decode_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def block_times(fn, calls_per_block, blocks, warmup, stream=None, warm_s=0.0):
    """Mean duration (ms) of one call of fn, for each of `blocks` blocks of
    `calls_per_block` back-to-back calls bracketed by one pair of HIP events
    on the stream fn launches on.  (A timing event recorded between two
    launches idles the GPU for ~10-15 us on this stack, so events never sit
    between the calls being timed.)  Before timing, fn runs `warmup` times
    and then until `warm_s` seconds have passed, so the blocks are timed at
    the clocks the GPU reaches under this load (after seconds of host-side
    input generation it starts from idle clocks)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(calls_per_block):
            fn()
        torch.cuda.synchronize()
    out = []
    for _ in range(blocks):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(calls_per_block):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / calls_per_block)
    return out


def graph_times(calls, reps, blocks=5):
    """Mean duration (ms) of one call when `reps` back-to-back calls (cycling
    through `calls`) are captured in one HIP graph and replayed, for each of
    `blocks` replays timed by a pair of HIP events: no host launch work sits
    between the kernels.  The calls write preallocated outputs."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:
        for c in calls:
            c()
        torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            calls[i % len(calls)]()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(blocks):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / reps)
    del g
    return out


def stream_probe():
    """ctypes handle of the HBM stream reference (libkvq_probe.so)."""
    import ctypes
    from ctypes import c_int, c_int64, c_void_p
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_compression_kvq_amd", "libkvq_probe.so"))
    lib.kvqprobe_stream_rw.restype = c_int
    lib.kvqprobe_stream_rw.argtypes = [c_void_p, c_int64, c_int, c_void_p, c_int, c_void_p, c_int,
                                       c_void_p]
    lib.kvqprobe_sketch_layout.restype = c_int
    lib.kvqprobe_sketch_layout.argtypes = [c_void_p, c_int64, c_int, c_void_p, c_void_p, c_int,
                                           c_void_p]
    return lib


def med(xs):
    s = sorted(xs)
    return s[len(s) // 2]


COLD_BYTES = 1 << 30     # rotate inputs over > 1 GiB: 4x the 256 MB last-level cache (MALL)
SECTIONS = ("copy", "tiny", "sweep", "llama", "qjl", "residual", "gqa")
# --config: one workload of the five (the decode step, or a set of component
# sections); "all" runs everything
CONFIGS = {"tiny": ("tiny",), "llama7b": ("llama",), "sweep": ("sweep",),
           "qjl": ("qjl", "residual", "gqa"), "decode": ()}


def components(K, si, torch, np, only=SECTIONS, use_graph=True):
    """GB/s of the INT8 (per row and per channel), INT4, QJL and two-stage
    kernels on their own workloads, cold (warmed-up clocks, cold caches): each
    timed call reads a different
    copy of its inputs, and the copies together exceed 1 GiB, so no call
    finds its inputs in the MALL or L2.  Outputs are preallocated (one set
    per component), so a call is the ctypes call and its launches only.
    Calls run back to back in blocks timed by one pair of HIP events; the
    median block's mean per call is reported ("ms", and the rates from it)
    with the fastest block's ("ms_min").  Kernels of a few microseconds (the
    Llama-7B layer, the QJL-cache scores) are also replayed from a HIP graph
    of back-to-back launches ("graph_ms"), which leaves the host's per-call
    launch work out."""
    res = {}
    dev = "cuda"

    def gbs(name, nbytes, calls, reps=20, flops=None, graph=False):
        """calls: list of zero-argument launches, one per input copy."""
        it = iter(range(10 ** 9))
        fn = lambda: calls[next(it) % len(calls)]()
        times = block_times(fn, max(reps, len(calls)), 5, 3, warm_s=0.25)
        ms = med(times)
        r = {"ms": round(ms, 4), "ms_min": round(min(times), 4), "GB/s": round(nbytes / ms / 1e6, 1),
             "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 3), "bytes": int(nbytes),
             "copies": len(calls)}
        if graph and use_graph:
            gt = graph_times(calls, len(calls) * max(1, 100 // len(calls)))
            gms = med(gt)
            r["graph_ms"] = round(gms, 4)
            r["graph_GB/s"] = round(nbytes / gms / 1e6, 1)
            r["graph_frac_hbm"] = round(nbytes / gms / 1e6 / HBM_PEAK_GBS, 3)
        if flops:
            r["TFLOP/s"] = round(flops / ms / 1e9, 1)
            r["frac_mfma_f16"] = round(flops / ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 3)
        res[name] = r
        log(f"  {name}: {r}")

    def ncopies(bytes_per_call):
        return max(1, -(-COLD_BYTES // int(bytes_per_call)) + 1)

    def like(outs):
        """A second set of outputs shaped like `outs` (a tensor or a tuple)."""
        if isinstance(outs, tuple):
            return tuple(torch.empty_like(t) for t in outs)
        return torch.empty_like(outs)

    if "copy" in only:
        # context: a plain device copy of 1 GiB (1 GiB read + 1 GiB written),
        # the practical rate of a stream that mixes reads and writes equally
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dsts = [torch.empty_like(src) for _ in range(2)]
        it_c = iter(range(10 ** 9))
        gbs("device_copy_1GiB", 2 * src.numel() * 4,
            [lambda: dsts[next(it_c) % 2].copy_(src)], reps=10)
        del src, dsts

    if "tiny" in only:
        # the correctness workload, timed for context (launch-bound): fp32 K
        # and V of one head, 512 tokens x 128; S 256 x 128 and 4 queries, fp32
        W, T1, d1, m1 = si.W_TINY, 512, 128, 256
        k1 = torch.from_numpy(si.kv_tensor(W, si.K, 1, 1, T1, d1, "f32")).to(dev).view(T1, d1)
        v1 = torch.from_numpy(si.kv_tensor(W, si.V, 1, 1, T1, d1, "f32")).to(dev).view(T1, d1)
        S1 = torch.from_numpy(si.projection(W, m1, d1, "f32")).to(dev)
        q1 = torch.from_numpy(si.queries(W, 1, 4, d1, "f32")).to(dev)
        kv1 = torch.stack([k1, v1]).view(-1, d1)
        c1 = K.quantize_int8(kv1)
        o1 = like(c1)
        gbs("tiny_quantize_kv_f32", 2 * T1 * d1 * 4 + 2 * T1 * (d1 + 4),
            [lambda: K.quantize_int8(kv1, out=o1)], graph=True)
        od1 = torch.empty_like(kv1)
        gbs("tiny_dequantize_kv_f32", 2 * T1 * (d1 + 4) + 2 * T1 * d1 * 4,
            [lambda: K.dequantize_int8(c1[0], c1[1], out=od1)], graph=True)
        kc1 = (c1[0][:T1].view(1, T1, d1), c1[1][:T1].view(1, T1))
        os1 = torch.empty((1, 4, T1), dtype=torch.float32, device=dev)
        gbs("tiny_scores_int8_4x512", T1 * (d1 + 4) + 4 * (d1 * 4 + T1 * 4),
            [lambda: K.scores_int8(q1, kc1[0], kc1[1], out=os1)], graph=True)
        sk1 = K.qjl_sketch(k1, S1)
        osk1 = like(sk1)
        gbs("tiny_qjl_sketch_f32_m256", T1 * d1 * 4 + T1 * (m1 // 8 + 2) + m1 * d1 * 4,
            [lambda: K.qjl_sketch(k1, S1, out=osk1)], flops=2.0 * T1 * d1 * m1, graph=True)
        b1, n1 = sk1[0].view(1, T1, m1 // 32), sk1[1].view(1, T1)
        gbs("tiny_qjl_scores_4x512", T1 * (m1 // 8 + 2) + 4 * (d1 * 4 + T1 * 4) + m1 * d1 * 4,
            [lambda: K.scores_qjl(q1, S1, b1, n1, out=os1)], graph=True)
        del k1, v1, S1, q1, kv1, c1, o1, od1, kc1, os1, sk1, osk1, b1, n1

    # INT8 round-trip error on the sweep (fp32 rows, N(0, 1)) and the
    # U(-1, 1) context row: max and mean |dequantize(quantize(x)) - x|
    acc = {}

    def round_trip_error(name, xv):
        codes, scales = K.quantize_int8(xv)
        err = (K.dequantize_int8(codes, scales) - xv).abs_()
        acc[name] = {"max_abs": float(err.max()),
                     "mean_abs": float(err.sum(dtype=torch.float64)) / err.numel()}
        del codes, scales, err

    if "sweep" in only:
        for nlog in (20, 24):
            x = torch.from_numpy(si.flat_rows(si.W_SWEEP, 1 << nlog, 128).reshape(-1)).to(dev)
            for d in (128, 1024, 8192):
                round_trip_error(f"f32_2^{nlog}_d{d}", x.view(-1, d))
        x = torch.from_numpy(si.flat_rows(si.W_SWEEP, 1 << 24, 128, dist="uniform").reshape(-1)).to(dev)
        round_trip_error("uniform_f32_2^24_d128", x.view(-1, 128))
        del x

        # element-count sweep, fp32 rows of d in {128, 1024, 8192}
        for nlog in (28, 30):
            n = 1 << nlog
            x = torch.from_numpy(si.flat_rows(si.W_SWEEP, n, 128).reshape(-1)).to(dev)
            xs = [x] + [x.clone() for _ in range(ncopies(4 * n) - 1)] if nlog < 30 else [x]
            for d in (128, 1024, 8192):
                rows = n // d
                views = [t.view(rows, d) for t in xs]
                round_trip_error(f"f32_2^{nlog}_d{d}", views[0])
                cs = [K.quantize_int8(v) for v in views]
                oq = like(cs[0])
                gbs(f"quantize_f32_2^{nlog}_d{d}", 4 * n + n + 4 * rows,
                    [lambda v=v: K.quantize_int8(v, out=oq) for v in views])
                del oq
                od = torch.empty((rows, d), dtype=torch.float32, device=dev)
                gbs(f"dequantize_f32_2^{nlog}_d{d}", n + 4 * rows + 4 * n,
                    [lambda c=c: K.dequantize_int8(c[0], c[1], out=od) for c in cs])
                del cs, od
                if d == 128:
                    # asymmetric group-wise INT4, groups of 32 and 128
                    for g in (32, 128):
                        c4 = [K.quantize_int4(v, g) for v in views]
                        o4 = like(c4[0])
                        gbs(f"quantize_int4_f32_2^{nlog}_d{d}_g{g}", 4 * n + n // 2 + 8 * (n // g),
                            [lambda v=v: K.quantize_int4(v, g, out=o4) for v in views])
                        del o4
                        od = torch.empty((rows, d), dtype=torch.float32, device=dev)
                        gbs(f"dequantize_int4_f32_2^{nlog}_d{d}_g{g}", n // 2 + 8 * (n // g) + 4 * n,
                            [lambda c=c: K.dequantize_int4(c[0], c[1], c[2], g, out=od) for c in c4])
                        del c4, od
            del x, xs
            torch.cuda.empty_cache()

    if "llama" in only:
        # Llama-7B-shaped layer, fp16: K and V quantized, dequantized, scored
        W = si.W_LLAMA_LAYER
        k = torch.from_numpy(si.kv_tensor(W, si.K, 1, 32, 4096, 128, "f16", outliers=True)).to(dev)
        v = torch.from_numpy(si.kv_tensor(W, si.V, 1, 32, 4096, 128, "f16")).to(dev)
        kv = torch.stack([k, v]).view(-1, 128)
        R = kv.shape[0]
        nc = ncopies(2 * R * 128)
        kvs = [kv] + [kv.clone() for _ in range(nc - 1)]
        cs = [K.quantize_int8(t) for t in kvs]
        oq = like(cs[0])
        gbs("llama_layer_quantize_kv_f16", 2 * R * 128 + R * 128 + 4 * R,
            [lambda t=t: K.quantize_int8(t, out=oq) for t in kvs], graph=True)
        od = torch.empty((R, 128), dtype=torch.float16, device=dev)
        gbs("llama_layer_dequantize_kv_f16", R * 128 + 4 * R + 2 * R * 128,
            [lambda c=c: K.dequantize_int8(c[0], c[1], torch.float16, out=od) for c in cs],
            graph=True)
        for g in (32, 128):
            c4 = [K.quantize_int4(t, g) for t in kvs]
            o4 = like(c4[0])
            gbs(f"llama_layer_quantize_int4_kv_f16_g{g}", 2 * R * 128 + R * 64 + 8 * R * (128 // g),
                [lambda t=t: K.quantize_int4(t, g, out=o4) for t in kvs], graph=True)
            gbs(f"llama_layer_dequantize_int4_kv_f16_g{g}", R * 64 + 8 * R * (128 // g) + 2 * R * 128,
                [lambda c=c: K.dequantize_int4(c[0], c[1], c[2], g, torch.float16, out=od)
                 for c in c4], graph=True)
            del c4, o4
        # per-channel INT8 keys (one scale per channel over a head's 4096 tokens)
        k3s = [t[: R // 2].view(32, 4096, 128) for t in kvs]
        cch = [K.quantize_int8_channel(t) for t in k3s]
        och = like(cch[0])
        half = R // 2
        gbs("llama_layer_quantize_int8_channel_k_f16", 2 * half * 128 + half * 128 + 4 * 32 * 128,
            [lambda t=t: K.quantize_int8_channel(t, out=och) for t in k3s], graph=True)
        odh = torch.empty((32, 4096, 128), dtype=torch.float16, device=dev)
        gbs("llama_layer_dequantize_int8_channel_k_f16", half * 128 + 4 * 32 * 128 + 2 * half * 128,
            [lambda c=c: K.dequantize_int8_channel(c[0], c[1], torch.float16, out=odh) for c in cch],
            graph=True)
        q = torch.from_numpy(si.queries(W, 32, 1, 128, "f16")).to(dev)
        osc = torch.empty((32, 1, 4096), dtype=torch.float32, device=dev)
        gbs("llama_layer_scores_int8_channel", 32 * 4096 * (128 + 4) + 32 * 128 * (2 + 4),
            [lambda c=c: K.scores_int8_channel(q, c[0], c[1], out=osc) for c in cch], graph=True)
        del k3s, cch, och, odh
        halves = [(c[0][: R // 2].view(32, 4096, 128), c[1][: R // 2].view(32, 4096)) for c in cs]
        gbs("llama_layer_scores_int8", 32 * 4096 * (128 + 4 + 4) + 32 * 128 * 2,
            [lambda h=h: K.scores_int8(q, h[0], h[1], out=osc) for h in halves], graph=True)
        # grouped-query attention, 4 query heads per KV head: one pass over the codes
        q4 = torch.from_numpy(si.queries(W, 32, 4, 128, "f16")).to(dev)
        osc4 = torch.empty((32, 4, 4096), dtype=torch.float32, device=dev)
        gbs("llama_layer_scores_int8_gqa4", 32 * 4096 * (128 + 4 + 4 * 4) + 32 * 4 * 128 * 2,
            [lambda h=h: K.scores_int8(q4, h[0], h[1], out=osc4) for h in halves], graph=True)
        # INT8 scores at a cache length where HBM, not launch latency, bounds
        # them: 32 heads x 262144 tokens x 128 (1.1 GB of codes), 1 and 4 queries
        Tl = 262144
        big = [(torch.randint(-127, 128, (32, Tl, 128), dtype=torch.int8, device=dev),
                torch.rand(32, Tl, device=dev)) for _ in range(2)]
        osl = torch.empty((32, 1, Tl), dtype=torch.float32, device=dev)
        gbs("scores_int8_32x262144x128", 32 * Tl * (128 + 4 + 4) + 32 * 128 * 2,
            [lambda c=c: K.scores_int8(q, c[0], c[1], out=osl) for c in big])
        osl4 = torch.empty((32, 4, Tl), dtype=torch.float32, device=dev)
        gbs("scores_int8_gqa4_32x262144x128", 32 * Tl * (128 + 4 + 4 * 4) + 32 * 4 * 128 * 2,
            [lambda c=c: K.scores_int8(q4, c[0], c[1], out=osl4) for c in big])
        del big, osl, osl4
        del k, v, kv, kvs, cs, halves, oq, od, osc, osc4
        torch.cuda.empty_cache()

    # QJL key cache: 8 x 32 x 8192 x 128 fp16, m = 256
    W = si.W_QJL_CACHE
    G, T, d, m = 256, 8192, 128, 256
    if "qjl" in only or "residual" in only:
        kk = torch.from_numpy(si.kv_tensor(W, si.K, 8, 32, T, d, "f16", outliers=True)).to(dev).view(-1, d)
        S = torch.from_numpy(si.projection(W, m, d, "f16")).to(dev)
        R = kk.shape[0]
        q = torch.from_numpy(si.queries(W, G, 1, d, "f16")).to(dev)
    if "qjl" in only:
        # practical HBM ceilings for the sketch's and the score's traffic
        # (a plain stream, no compression work): rows of 256 B read and 32 B
        # written, and rows of 32 B read only, over the same row count
        probe = stream_probe()
        sink = torch.zeros(4096, dtype=torch.uint8, device=dev)
        src = [torch.empty(R * 256, dtype=torch.uint8, device=dev).fill_(i + 1)
               for i in range(ncopies(R * 256))]
        dst = torch.empty(R * 32, dtype=torch.uint8, device=dev)
        nblk = 16 * torch.cuda.get_device_properties(0).multi_processor_count

        def run_probe(a, rd_log2, b, wr16):
            rc = probe.kvqprobe_stream_rw(a.data_ptr(), R, rd_log2, b.data_ptr() if b is not None
                                          else None, wr16, sink.data_ptr(), nblk,
                                          torch.cuda.current_stream().cuda_stream)
            assert rc == 0, rc

        gbs("stream_ref_read256_write32_B_per_row", R * (256 + 32),
            [lambda a=a: run_probe(a, 4, dst, 2) for a in src])
        src32 = [a[: R * 32] for a in src]
        gbs("stream_ref_read32_B_per_row", R * 32,
            [lambda a=a: run_probe(a, 1, None, 0) for a in src32], graph=True)
        # the sketch's memory side alone: its grid, 32-row wave tiles, ring of
        # two and writes (32 B words + 2 B norm per row), no multiplies; the
        # keys read in the matrix-core operand layout (32 rows x 32 B per
        # load instruction, as the sketch reads them) or as whole lines
        nrm = torch.empty(R, dtype=torch.int16, device=dev)
        ncu = torch.cuda.get_device_properties(0).multi_processor_count

        def run_layout(a, layout):
            rc = probe.kvqprobe_sketch_layout(a.data_ptr(), R, layout, dst.data_ptr(), nrm.data_ptr(),
                                              ncu, torch.cuda.current_stream().cuda_stream)
            assert rc == 0, rc

        for layout, nm in ((0, "operand_layout"), (1, "whole_lines"), (2, "whole_lines_nt")):
            gbs(f"stream_ref_sketch_grid_{nm}", R * (256 + 32 + 2),
                [lambda a=a, layout=layout: run_layout(a, layout) for a in src])
        del src, src32, dst, sink, nrm
        kks = [kk] + [kk.clone() for _ in range(ncopies(R * d * 2) - 1)]
        sk = [K.qjl_sketch(t, S) for t in kks]
        osk = like(sk[0])
        gbs("qjl_sketch_f16_m256", R * d * 2 + R * (m // 8) + 2 * R + m * d * 2,
            [lambda t=t: K.qjl_sketch(t, S, out=osk) for t in kks], flops=2.0 * R * d * m)
        del kks, osk
        b3 = [(b.view(G, T, m // 32), n.view(G, T)) for b, n in sk]
        while len(b3) < ncopies(R * (m // 8 + 2)):
            b3.append((b3[0][0].clone(), b3[0][1].clone()))
        oqs = torch.empty((G, 1, T), dtype=torch.float32, device=dev)
        gbs("qjl_scores_f16_m256", R * (m // 8 + 2 + 4) + G * d * 2 + m * d * 2,
            [lambda bn=bn: K.scores_qjl(q, S, bn[0], bn[1], out=oqs) for bn in b3], graph=True)
        res["qjl_scores_f16_m256"]["scores/s"] = round(R / res["qjl_scores_f16_m256"]["ms"] * 1e3, 1)
        # grouped-query attention, 4 query heads per KV head: one pass over the sign words
        q4 = torch.from_numpy(si.queries(W, G, 4, d, "f16")).to(dev)
        oqs4 = torch.empty((G, 4, T), dtype=torch.float32, device=dev)
        gbs("qjl_scores_gqa4_f16_m256", R * (m // 8 + 2 + 4 * 4) + G * 4 * d * 2 + m * d * 2,
            [lambda bn=bn: K.scores_qjl(q4, S, bn[0], bn[1], out=oqs4) for bn in b3], graph=True)
        res["qjl_scores_gqa4_f16_m256"]["scores/s"] = round(
            4 * R / res["qjl_scores_gqa4_f16_m256"]["ms"] * 1e3, 1)
        del sk, b3, oqs, oqs4
    if "residual" in only:
        # two-stage keys: INT4 (groups of 32) and the QJL sketch of its residual
        g4 = 32
        per_tok = d // 2 + 8 * (d // g4) + m // 8 + 2
        kks = [kk] + [kk.clone() for _ in range(ncopies(R * d * 2) - 1)]
        first = K.residual_sketch(kk, S, g4)
        ors = like(first)
        gbs("residual_sketch_f16_m256_g32", R * d * 2 + R * per_tok + m * d * 2,
            [lambda t=t: K.residual_sketch(t, S, g4, out=ors) for t in kks], flops=2.0 * R * d * m)
        del kks, ors
        c4, s4, z4, b4, n4 = first
        st = [(c4.view(G, T, d // 2), s4.view(G, T, d // g4), z4.view(G, T, d // g4),
               b4.view(G, T, m // 32), n4.view(G, T))]
        while len(st) < ncopies(R * per_tok):
            st.append(tuple(x.clone() for x in st[0]))
        ors = torch.empty((G, 1, T), dtype=torch.float32, device=dev)
        gbs("residual_scores_f16_m256_g32", R * (per_tok + 4) + G * d * 2 + m * d * 2,
            [lambda a=a: K.scores_residual(q, S, *a, g4, out=ors) for a in st])
        res["residual_scores_f16_m256_g32"]["scores/s"] = round(
            R / res["residual_scores_f16_m256_g32"]["ms"] * 1e3, 1)
        del st, first, ors
    if "qjl" in only or "residual" in only:
        del kk, S, q
        torch.cuda.empty_cache()

    if "gqa" in only:
        # grouped-query decode: 128 KV heads (16 x 8) x 32768 tokens, 4 query
        # heads per KV head (m = 256, d = 128), against the same 4 queries
        # decoded one at a time; cache from the bench's decode generator recipe
        # (fp16 N(0,1) keys and values, QJL keys, INT8 values) on 16 x 8 heads
        Gk, Tq, nqg = 128, 32768, 4
        kbits_, knorm_, vcode_, vscal_ = [], [], [], []
        Sg = torch.from_numpy(si.projection(si.W_DECODE, m, d, "f16")).to(dev)
        for g0 in range(0, Gk, 16):
            kk_ = torch.from_numpy(si.stream(si.W_DECODE, si.K, 16 * Tq * d, "f16",
                                             start=g0 * Tq * d)).to(dev).view(-1, d)
            vv_ = torch.from_numpy(si.stream(si.W_DECODE, si.V, 16 * Tq * d, "f16",
                                             start=g0 * Tq * d)).to(dev).view(-1, d)
            b_, n_ = K.qjl_sketch(kk_, Sg)
            c_, s_ = K.quantize_int8(vv_)
            kbits_.append(b_); knorm_.append(n_); vcode_.append(c_); vscal_.append(s_)
            del kk_, vv_
        kbg = torch.cat(kbits_).view(Gk, Tq, m // 32)
        kng = torch.cat(knorm_).view(Gk, Tq)
        vcg = torch.cat(vcode_).view(Gk, Tq, d)
        vsg = torch.cat(vscal_).view(Gk, Tq)
        del kbits_, knorm_, vcode_, vscal_
        qg = torch.from_numpy(si.queries(si.W_DECODE, Gk, nqg, d, "f16")).to(dev)
        wsg = torch.empty(K.decode_gqa_workspace_bytes(Gk, nqg, Tq, d, m), dtype=torch.uint8, device=dev)
        og = torch.empty((Gk, nqg, d), dtype=torch.float32, device=dev)
        gbs("decode_gqa4_128x32768", Gk * Tq * (m // 8 + 2 + d + 4) + Gk * nqg * d * (2 + 4),
            [lambda: K.decode_qjl_int8_gqa(qg, Sg, kbg, kng, vcg, vsg, workspace=wsg, out=og)],
            reps=10)
        res["decode_gqa4_128x32768"]["scores/s"] = round(
            Gk * nqg * Tq / res["decode_gqa4_128x32768"]["ms"] * 1e3, 1)
        qs1 = [qg[:, j].contiguous() for j in range(nqg)]
        ws1 = torch.empty(K.decode_workspace_bytes(Gk, Tq, d, m), dtype=torch.uint8, device=dev)
        o1 = torch.empty((Gk, d), dtype=torch.float32, device=dev)
        gbs("decode_4x1query_128x32768", 4 * (Gk * Tq * (m // 8 + 2 + d + 4) + Gk * d * (2 + 4)),
            [lambda: [K.decode_qjl_int8(qq, Sg, kbg, kng, vcg, vsg, workspace=ws1, out=o1)
                      for qq in qs1]], reps=10)
        res["decode_4x1query_128x32768"]["scores/s"] = round(
            Gk * nqg * Tq / res["decode_4x1query_128x32768"]["ms"] * 1e3, 1)
        del kbg, kng, vcg, vsg, qg, wsg, og, ws1, o1
        torch.cuda.empty_cache()
    if acc:
        res["int8_round_trip_error"] = acc
        log(f"  int8_round_trip_error: {acc}")
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Host threads the oracle may use: the process's CPU affinity, capped at
    16 (the host cores set aside per GPU on a one-GPU MI355X host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _timed_pool(fn, items, threads):
    """Wall time of fn over items on a pool of `threads` threads (numpy
    releases the GIL inside its array operations; BLAS is held to one thread
    per call by the caller)."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fn, items))
    return time.perf_counter() - t0


def cpu_baseline(si, np, seconds, gpu_quantize_ms=None):
    """The fp64 oracle, timed on the host's cores on bounded samples of two
    workloads (the oracle as it stands: a correctness reference, not a tuned
    CPU kernel):
      * the decode step (16 x 32 x 32768 x 128, m = 256): whole (batch, head)
        groups, on one thread, then on every thread of the process's CPU
        affinity (one group per task);
      * INT8 quantize of the 2^28-element fp32 sweep at d = 128: 2^22-element
        row blocks, one thread and every thread; with the GPU kernel's time
        for the whole 2^28 elements, the GPU/CPU ratio is printed beside the
        INT8 page's "up to 1,694x" (context only).
    Input generation and cache building are outside the timed regions."""
    from threadpoolctl import threadpool_limits
    from oracle import decode as OD, int8 as OI, qjl as OQ
    nth = cpu_threads()
    W, B, H, T, d, m = si.W_DECODE, 16, 32, 32768, 128, 256
    S = si.projection(W, m, d, "f16")
    q = si.queries(W, B * H, 1, d, "f16")[:, 0]
    lam = 1.0 / math.sqrt(d)

    def group(g):
        # group g is rows [g * T, (g + 1) * T) of the [B*H*T, d] tensors
        k = si.stream(W, si.K, T * d, "f16", start=g * T * d, workers=1).reshape(T, d)
        v = si.stream(W, si.V, T * d, "f16", start=g * T * d, workers=1).reshape(T, d)
        kw, kn = OQ.qjl_sketch(k, S)
        vc, vs = OI.quantize_int8(v)
        return kw[None], kn[None], vc[None], vs[None]

    def decode(args):
        g, (kw, kn, vc, vs) = args
        OD.decode_qjl_int8(q[g:g + 1], S, kw, kn, vc, vs, lam)

    with threadpool_limits(1):
        # one thread: groups until `seconds` of compute (at least 2 groups)
        done, spent = 0, 0.0
        while done < B * H and (spent < seconds or done < 2):
            c = group(done)
            t0 = time.perf_counter()
            decode((done, c))
            spent += time.perf_counter() - t0
            done += 1
        one = {"value": round(done * T / spent, 1), "unit": "scores/s", "cores": 1,
               "seconds": round(spent, 2),
               "sample": f"{done} of {B * H} (batch, head) groups x {T} tokens, one decode query each"}
        # every thread: enough groups for about `seconds` of wall time
        n = min(B * H, max(nth, int(nth * seconds * one["value"] / T)))
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=nth) as ex:     # cache build, untimed
            caches = list(zip(range(n), ex.map(group, range(n))))
        wall = _timed_pool(decode, caches, nth)
        del caches
        allc = {"value": round(n * T / wall, 1), "unit": "scores/s", "cores": nth,
                "seconds": round(wall, 2),
                "sample": f"{n} of {B * H} (batch, head) groups x {T} tokens, one decode query each, "
                          f"one group per task on {nth} threads"}

        # INT8 quantize, fp32 sweep 2^28 elements as rows of 128
        n_el, dq = 1 << 28, 128
        blk = 1 << 22
        nblk_total = n_el // blk
        x0 = si.flat_rows(si.W_SWEEP, blk, dq, rows=range(0, blk // dq))
        t0 = time.perf_counter()
        nb = 0
        while nb < nblk_total and (time.perf_counter() - t0 < seconds / 2 or nb < 1):
            OI.quantize_int8(x0)
            nb += 1
        t1 = time.perf_counter() - t0
        bytes_per_el = 4 + 1 + 4 / dq
        q1 = {"value": round(nb * blk * bytes_per_el / t1 / 1e9, 3), "unit": "GB/s", "cores": 1,
              "seconds": round(t1, 2),
              "sample": f"{nb} of the {nblk_total} 2^22-element blocks of the 2^28 sweep (d = 128)"}
        nb_all = min(nblk_total, max(nth, int(nth * seconds / 2 / (t1 / nb))))
        blocks = [si.flat_rows(si.W_SWEEP, n_el, dq, rows=range(i * (blk // dq), (i + 1) * (blk // dq)))
                  for i in range(min(nb_all, nth))]
        wall = _timed_pool(lambda i: OI.quantize_int8(blocks[i % len(blocks)]), range(nb_all), nth)
        qa = {"value": round(nb_all * blk * bytes_per_el / wall / 1e9, 3), "unit": "GB/s",
              "cores": nth, "seconds": round(wall, 2),
              "sample": f"{nb_all} 2^22-element blocks of the 2^28 sweep (d = 128), one per task "
                        f"on {nth} threads"}
        del blocks
    quant = {"one_core": q1, "all_cores": qa}
    if gpu_quantize_ms:
        gpu_gbs = n_el * bytes_per_el / (gpu_quantize_ms / 1e3) / 1e9
        quant["gpu_GB/s"] = round(gpu_gbs, 1)
        quant["gpu_over_cpu"] = {"one_core": round(gpu_gbs / q1["value"], 1),
                                 "all_cores": round(gpu_gbs / qa["value"], 1),
                                 "context": "the INT8 page (arXiv 2601.04719, Abstract) reports up "
                                            "to 1,694x over its CPU baselines, hardware not stated"}
    return {"value": allc["value"], "unit": "scores/s", "cores": nth, "kind": "oracle",
            "sample": allc["sample"] + "; fp64 numpy oracle (decode of the long-context workload)",
            "cpu_model": cpu_model(), "one_core": one, "all_cores": allc,
            "int8_quantize_2^28_d128": quant}


PROVENANCE = {
    "measured": ["ms_per_step (wall clock around the timed steps)", "graph_ms_per_step",
                 "roofline.avg_launch_ms (HIP events)", "roofline.traffic (rocprofv3 FETCH_SIZE "
                 "and WRITE_SIZE, scaled by a known copy)", "components.*.ms, ms_min, graph_ms "
                 "(HIP events)", "cpu_baseline.*.seconds"],
    "derived": ["value = scores per step / ms_per_step", "roofline.achieved, frac = algorithmic "
                "bytes / avg_launch_ms", "components.*.GB/s, frac_hbm, TFLOP/s, frac_mfma_f16, "
                "scores/s = algorithmic bytes, flops or scores / ms", "cpu_baseline.*.value = work "
                "/ seconds", "cpu_baseline.int8_quantize_2^28_d128.gpu_over_cpu"],
}


DECODE_KERNELS = ("qjl_project_kernel", "decode_split_kernel", "decode_merge_kernel")


def traffic_summary(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """HBM bytes per kvq_decode_qjl_int8 launch from rocprofv3 counters:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, mean over the run's
    dispatches of each decode kernel) summed over the launch's three kernels,
    each scaled by known bytes / counter bytes of a 1 GiB device copy."""
    import csv
    from collections import defaultdict

    def per_kernel(path, counter):
        acc = defaultdict(list)
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] == counter:
                    acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}, {k: len(v) for k, v in acc.items()}

    def copy_scale(path, counter):
        vals, _ = per_kernel(path, counter)
        kib = [v for k, v in vals.items() if "copyBuffer" in k]
        return (1 << 30) / 1024 / kib[0]

    f, nf = per_kernel(fetch_csv, "FETCH_SIZE")
    w, _ = per_kernel(write_csv, "WRITE_SIZE")
    fs, ws = copy_scale(cal_fetch_csv, "FETCH_SIZE"), copy_scale(cal_write_csv, "WRITE_SIZE")
    kernels = {}
    for k in f:
        if any(n in k for n in DECODE_KERNELS):
            kernels[k] = {"fetch_kib": round(f[k], 1), "write_kib": round(w.get(k, 0.0), 1),
                          "dispatches": nf[k]}
    fk = sum(v["fetch_kib"] for v in kernels.values())
    wk = sum(v["write_kib"] for v in kernels.values())
    hbm = int(round(fk * 1024 * fs + wk * 1024 * ws))
    G, T, d, m = 512, 32768, 128, 256
    alg = G * T * (m // 8 + 2 + d + 4) + G * d * 2 + m * d * 2 + G * d * 4
    out = {"source_sha": decode_source_hash(), "hbm_bytes_per_launch": hbm,
           "alg_bytes_per_launch": alg, "traffic_over_alg": round(hbm / alg, 3),
           "fetch_kib_per_launch": round(fk, 1), "write_kib_per_launch": round(wk, 1),
           "fetch_scale": round(fs, 3), "write_scale": round(ws, 3), "kernels": kernels,
           "how": "rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (KiB per dispatch, mean over the "
                  "bench's decode dispatches), each scaled by the ratio of a 1 GiB device copy's "
                  "known bytes to the same counter (bench.py --traffic-summary)"}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def main():
    args = parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 28                                   # 2^28 fp32 = 1 GiB each way
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))
        return

    import kv_cache_compression_kvq_amd as K
    import synth_inputs as si

    torch.cuda.set_device(0)

    only = tuple(x for x in args.only.split(",") if x)
    if args.config != "all":
        only = CONFIGS[args.config] + (("copy",) if args.config == "sweep" else ())
        args.no_decode = args.config != "decode"
        args.no_components = args.config == "decode"
    bad = [x for x in only if x not in SECTIONS]
    if bad:
        print(f"unknown section(s) {bad}; sections: {', '.join(SECTIONS)}", file=sys.stderr)
        sys.exit(2)

    value = ms_step = graph_ms_step = roofline = None
    if not args.no_decode:
        value, ms_step, graph_ms_step, roofline = decode_step(K, si, torch, args)

    comp = None
    if not args.no_components:
        torch.cuda.empty_cache()
        log("bench: components")
        comp = components(K, si, torch, np, only, not args.no_graph)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        gq = (comp or {}).get("quantize_f32_2^28_d128", {}).get("ms")
        cpu = cpu_baseline(si, np, args.cpu_seconds, gq)

    line = {
        "metric": "KV quantize/dequant HBM GB/s (% of peak); QJL+INT8 decode scores/sec",
        "value": None if value is None else round(value, 1),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": None if ms_step is None else round(ms_step, 4),
        "graph_ms_per_step": None if graph_ms_step is None else round(graph_ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode step over a QJL-key / INT8-value cache: batch 16 x 32 heads "
                               "x 32768 tokens x d 128, m 256, 1 fp16 query per head, newest token "
                               "compressed in-step",
                   "global_batch": 16, "seq_len": 32768, "heads": 32, "head_dim": 128, "qjl_m": 256,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "components": comp,
        "provenance": PROVENANCE,
    }
    print(json.dumps(line), flush=True)


def decode_step(K, si, torch, args):
    """The headline: K decode steps timed back to back (see the module
    docstring).  Returns (scores/s, ms per step, ms per step from a HIP graph
    replay, roofline of the decode launch)."""
    dev = "cuda"
    W, B, H, T, d, m = si.W_DECODE, 16, 32, 32768, 128, 256
    G = B * H
    lam = 1.0 / math.sqrt(d)

    log("bench: generating the decode cache (fp16 K, V ~ N(0,1), 16x32x32768x128)")
    t0 = time.time()
    k = torch.from_numpy(si.kv_tensor(W, si.K, B, H, T, d, "f16")).to(dev).view(G, T, d)
    S = torch.from_numpy(si.projection(W, m, d, "f16")).to(dev)
    kbits, knorms = K.qjl_sketch(k, S)
    del k
    v = torch.from_numpy(si.kv_tensor(W, si.V, B, H, T, d, "f16")).to(dev).view(G, T, d)
    vcodes, vscales = K.quantize_int8(v)
    del v
    torch.cuda.empty_cache()
    q = torch.from_numpy(si.queries(W, G, 1, d, "f16")).to(dev).view(G, d)
    # the newest token of every head (its own streams: tensor ids 6, 7)
    k_new = torch.from_numpy(si.stream(W, 6, G * d, "f16")).to(dev).view(G, d)
    v_new = torch.from_numpy(si.stream(W, 7, G * d, "f16")).to(dev).view(G, d)
    ws = torch.empty(max(16, K.decode_workspace_bytes(G, T, d, m)), dtype=torch.uint8, device=dev)
    out = torch.empty((G, d), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"bench: cache ready in {time.time() - t0:.1f} s")

    # One step: compress the newest token of every head into position T - 1
    # of the cache (one launch), then decode (three launches).  Launched
    # eagerly: the host enqueues a step in far less time than the GPU runs
    # it, so consecutive kernels start back to back (a HIP graph replay would
    # add a ~10 us gap at every graph boundary on this stack).
    def step():
        K.cache_append(k_new, v_new, S, kbits, knorms, vcodes, vscales, T - 1)
        K.decode_qjl_int8(q, S, kbits, knorms, vcodes, vscales, lam, workspace=ws, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    # Timed region: K steps back to back.  HIP events sit only at its ends: a
    # timing event recorded between two launches idles the GPU for ~15 us.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    step_ev_ms = ev0.elapsed_time(ev1) / args.steps

    # Decode launch duration for the roofline: K decode launches back to back
    # between one pair of HIP events on the launch stream.
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.steps):
        K.decode_qjl_int8(q, S, kbits, knorms, vcodes, vscales, lam, workspace=ws, out=out)
    d1.record(stream)
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / args.steps
    ms_step = elapsed * 1e3 / args.steps

    # The same step captured 20 times in one HIP graph and replayed: the
    # per-step time with host launch overhead taken out (reported beside the
    # eager figure, which is `value`).
    graph = torch.cuda.CUDAGraph()
    graph_steps = 20
    with torch.cuda.graph(graph):
        for _ in range(graph_steps):
            step()
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    t_g = time.perf_counter()
    for _ in range(5):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms_step = (time.perf_counter() - t_g) * 1e3 / (5 * graph_steps)
    del graph
    scores = G * T
    value = scores / (ms_step / 1e3)

    alg_bytes = (G * T * (m // 8 + 2 + d + 4)       # sign words, norm, value codes, value scale
                 + G * d * 2 + m * d * 2 + G * d * 4)  # queries, S, output
    achieved = alg_bytes / (dec_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(alg_bytes),
                "kernel": "kvq_decode_qjl_int8 (qjl_project_kernel + decode_split_kernel + decode_merge_kernel)",
                "alg_bytes_per_launch": alg_bytes, "avg_launch_ms": round(dec_ms, 4),
                "launch_timing": f"{args.steps} back-to-back launches between HIP events"}
    log(f"bench: graph replay {graph_ms_step:.3f} ms/step")
    log(f"bench: {args.steps} steps, {ms_step:.3f} ms/step (events {step_ev_ms:.3f}), "
        f"decode {dec_ms:.3f} ms "
        f"({achieved:.0f} GB/s)")
    del kbits, knorms, vcodes, vscales, k_new, v_new, ws, out, q, S
    return value, ms_step, graph_ms_step, roofline


if __name__ == "__main__":
    main()
