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

Also reported (``components``): HBM GB/s of quantize / dequantize on the
element-count sweep (2^28 and 2^30 fp32), the Llama-7B-layer INT8 path, and
the QJL-cache sketch and score, each timed with HIP events on the stream the
kernels run on.  ``cpu_baseline`` times the fp64 oracle on a bounded sample
of the same decode workload.

    python bench.py [--gpus 1] [--steps 50] [--warmup 1000] [--no-components]

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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
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


def block_times(fn, calls_per_block, blocks, warmup, stream=None):
    """Mean duration (ms) of one call of fn, for each of `blocks` blocks of
    `calls_per_block` back-to-back calls bracketed by one pair of HIP events
    on the stream fn launches on.  (A timing event recorded between two
    launches idles the GPU for ~10-15 us on this stack, so events never sit
    between the calls being timed.)"""
    import torch
    for _ in range(warmup):
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


def med(xs):
    s = sorted(xs)
    return s[len(s) // 2]


COLD_BYTES = 1 << 30     # rotate inputs over > 1 GiB: 4x the 256 MB last-level cache (MALL)


def components(K, si, torch, np):
    """GB/s of the INT8 (per row and per channel), INT4, QJL and two-stage
    kernels on their own workloads, cold: each timed call reads a different
    copy of its inputs, and the copies together
    exceed 1 GiB, so no call finds its inputs in the MALL or L2.  Calls run
    back to back in blocks timed by one pair of HIP events; the median block's
    mean per call is reported ("ms", and the rates from it) with the fastest
    block's ("ms_min")."""
    res = {}
    dev = "cuda"

    def gbs(name, nbytes, calls, reps=20, flops=None):
        """calls: list of zero-argument launches, one per input copy."""
        it = iter(range(10 ** 9))
        fn = lambda: calls[next(it) % len(calls)]()
        times = block_times(fn, max(reps, len(calls)), 5, 3)
        ms = med(times)
        r = {"ms": round(ms, 4), "ms_min": round(min(times), 4), "GB/s": round(nbytes / ms / 1e6, 1),
             "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 3), "bytes": int(nbytes),
             "copies": len(calls)}
        if flops:
            r["TFLOP/s"] = round(flops / ms / 1e9, 1)
            r["frac_mfma_f16"] = round(flops / ms / 1e9 / MFMA_F16_PEAK_TFLOPS, 3)
        res[name] = r
        log(f"  {name}: {r}")

    def ncopies(bytes_per_call):
        return max(1, -(-COLD_BYTES // int(bytes_per_call)) + 1)

    # context: a plain device copy of 1 GiB (1 GiB read + 1 GiB written), the
    # practical rate of a stream that mixes reads and writes equally
    src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    dsts = [torch.empty_like(src) for _ in range(2)]
    it_c = iter(range(10 ** 9))
    gbs("device_copy_1GiB", 2 * src.numel() * 4,
        [lambda: dsts[next(it_c) % 2].copy_(src)], reps=10)
    del src, dsts

    # INT8 round-trip error on the sweep (fp32 rows, N(0, 1)) and the
    # U(-1, 1) context row: max and mean |dequantize(quantize(x)) - x|
    acc = {}

    def round_trip_error(name, xv):
        codes, scales = K.quantize_int8(xv)
        err = (K.dequantize_int8(codes, scales) - xv).abs_()
        acc[name] = {"max_abs": float(err.max()),
                     "mean_abs": float(err.sum(dtype=torch.float64)) / err.numel()}
        del codes, scales, err

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
            gbs(f"quantize_f32_2^{nlog}_d{d}", 4 * n + n + 4 * rows,
                [lambda v=v: K.quantize_int8(v) for v in views])
            gbs(f"dequantize_f32_2^{nlog}_d{d}", n + 4 * rows + 4 * n,
                [lambda c=c: K.dequantize_int8(c[0], c[1]) for c in cs])
            del cs
            if d == 128:
                # asymmetric group-wise INT4, groups of 32 and 128
                for g in (32, 128):
                    c4 = [K.quantize_int4(v, g) for v in views]
                    gbs(f"quantize_int4_f32_2^{nlog}_d{d}_g{g}", 4 * n + n // 2 + 8 * (n // g),
                        [lambda v=v: K.quantize_int4(v, g) for v in views])
                    gbs(f"dequantize_int4_f32_2^{nlog}_d{d}_g{g}", n // 2 + 8 * (n // g) + 4 * n,
                        [lambda c=c: K.dequantize_int4(c[0], c[1], c[2], g) for c in c4])
                    del c4
        del x, xs
        torch.cuda.empty_cache()

    # Llama-7B-shaped layer, fp16: K and V quantized, dequantized, scored
    W = si.W_LLAMA_LAYER
    k = torch.from_numpy(si.kv_tensor(W, si.K, 1, 32, 4096, 128, "f16", outliers=True)).to(dev)
    v = torch.from_numpy(si.kv_tensor(W, si.V, 1, 32, 4096, 128, "f16")).to(dev)
    kv = torch.stack([k, v]).view(-1, 128)
    R = kv.shape[0]
    nc = ncopies(2 * R * 128)
    kvs = [kv] + [kv.clone() for _ in range(nc - 1)]
    cs = [K.quantize_int8(t) for t in kvs]
    gbs("llama_layer_quantize_kv_f16", 2 * R * 128 + R * 128 + 4 * R,
        [lambda t=t: K.quantize_int8(t) for t in kvs])
    gbs("llama_layer_dequantize_kv_f16", R * 128 + 4 * R + 2 * R * 128,
        [lambda c=c: K.dequantize_int8(c[0], c[1], torch.float16) for c in cs])
    for g in (32, 128):
        c4 = [K.quantize_int4(t, g) for t in kvs]
        gbs(f"llama_layer_quantize_int4_kv_f16_g{g}", 2 * R * 128 + R * 64 + 8 * R * (128 // g),
            [lambda t=t: K.quantize_int4(t, g) for t in kvs])
        gbs(f"llama_layer_dequantize_int4_kv_f16_g{g}", R * 64 + 8 * R * (128 // g) + 2 * R * 128,
            [lambda c=c: K.dequantize_int4(c[0], c[1], c[2], g, torch.float16) for c in c4])
        del c4
    # per-channel INT8 keys (one scale per channel over a head's 4096 tokens)
    k3s = [t[: R // 2].view(32, 4096, 128) for t in kvs]
    cch = [K.quantize_int8_channel(t) for t in k3s]
    half = R // 2
    gbs("llama_layer_quantize_int8_channel_k_f16", 2 * half * 128 + half * 128 + 4 * 32 * 128,
        [lambda t=t: K.quantize_int8_channel(t) for t in k3s])
    gbs("llama_layer_dequantize_int8_channel_k_f16", half * 128 + 4 * 32 * 128 + 2 * half * 128,
        [lambda c=c: K.dequantize_int8_channel(c[0], c[1], torch.float16) for c in cch])
    qch = torch.from_numpy(si.queries(W, 32, 1, 128, "f16")).to(dev)
    gbs("llama_layer_scores_int8_channel", 32 * 4096 * (128 + 4) + 32 * 128 * (2 + 4),
        [lambda c=c: K.scores_int8_channel(qch, c[0], c[1]) for c in cch])
    del k3s, cch
    q = torch.from_numpy(si.queries(W, 32, 1, 128, "f16")).to(dev)
    halves = [(c[0][: R // 2].view(32, 4096, 128), c[1][: R // 2].view(32, 4096)) for c in cs]
    gbs("llama_layer_scores_int8", 32 * 4096 * (128 + 4 + 4) + 32 * 128 * 2,
        [lambda h=h: K.scores_int8(q, h[0], h[1]) for h in halves])
    # grouped-query attention, 4 query heads per KV head: one pass over the codes
    q4 = torch.from_numpy(si.queries(W, 32, 4, 128, "f16")).to(dev)
    gbs("llama_layer_scores_int8_gqa4", 32 * 4096 * (128 + 4 + 4 * 4) + 32 * 4 * 128 * 2,
        [lambda h=h: K.scores_int8(q4, h[0], h[1]) for h in halves])
    # INT8 scores at a cache length where HBM, not launch latency, bounds
    # them: 32 heads x 262144 tokens x 128 (1.1 GB of codes), 1 and 4 queries
    Tl = 262144
    big = [(torch.randint(-127, 128, (32, Tl, 128), dtype=torch.int8, device=dev),
            torch.rand(32, Tl, device=dev)) for _ in range(2)]
    gbs("scores_int8_32x262144x128", 32 * Tl * (128 + 4 + 4) + 32 * 128 * 2,
        [lambda c=c: K.scores_int8(q, c[0], c[1]) for c in big])
    gbs("scores_int8_gqa4_32x262144x128", 32 * Tl * (128 + 4 + 4 * 4) + 32 * 4 * 128 * 2,
        [lambda c=c: K.scores_int8(q4, c[0], c[1]) for c in big])
    del big
    del k, v, kv, kvs, cs, halves
    torch.cuda.empty_cache()

    # QJL key cache: 8 x 32 x 8192 x 128 fp16, m = 256
    W = si.W_QJL_CACHE
    G, T, d, m = 256, 8192, 128, 256
    kk = torch.from_numpy(si.kv_tensor(W, si.K, 8, 32, T, d, "f16", outliers=True)).to(dev).view(-1, d)
    S = torch.from_numpy(si.projection(W, m, d, "f16")).to(dev)
    R = kk.shape[0]
    kks = [kk] + [kk.clone() for _ in range(ncopies(R * d * 2) - 1)]
    sk = [K.qjl_sketch(t, S) for t in kks]
    gbs("qjl_sketch_f16_m256", R * d * 2 + R * (m // 8) + 2 * R + m * d * 2,
        [lambda t=t: K.qjl_sketch(t, S) for t in kks], flops=2.0 * R * d * m)
    del kks
    q = torch.from_numpy(si.queries(W, G, 1, d, "f16")).to(dev)
    b3 = [(b.view(G, T, m // 32), n.view(G, T)) for b, n in sk]
    while len(b3) < ncopies(R * (m // 8 + 2)):
        b3.append((b3[0][0].clone(), b3[0][1].clone()))
    gbs("qjl_scores_f16_m256", R * (m // 8 + 2 + 4) + G * d * 2 + m * d * 2,
        [lambda bn=bn: K.scores_qjl(q, S, bn[0], bn[1]) for bn in b3])
    res["qjl_scores_f16_m256"]["scores/s"] = round(R / res["qjl_scores_f16_m256"]["ms"] * 1e3, 1)
    # grouped-query attention, 4 query heads per KV head: one pass over the sign words
    q4 = torch.from_numpy(si.queries(W, G, 4, d, "f16")).to(dev)
    gbs("qjl_scores_gqa4_f16_m256", R * (m // 8 + 2 + 4 * 4) + G * 4 * d * 2 + m * d * 2,
        [lambda bn=bn: K.scores_qjl(q4, S, bn[0], bn[1]) for bn in b3])
    res["qjl_scores_gqa4_f16_m256"]["scores/s"] = round(
        4 * R / res["qjl_scores_gqa4_f16_m256"]["ms"] * 1e3, 1)
    # two-stage keys: INT4 (groups of 32) and the QJL sketch of its residual
    g4 = 32
    per_tok = d // 2 + 8 * (d // g4) + m // 8 + 2
    kks = [kk] + [kk.clone() for _ in range(ncopies(R * d * 2) - 1)]
    first = K.residual_sketch(kk, S, g4)
    gbs("residual_sketch_f16_m256_g32", R * d * 2 + R * per_tok + m * d * 2,
        [lambda t=t: K.residual_sketch(t, S, g4) for t in kks], flops=2.0 * R * d * m)
    del kks
    c4, s4, z4, b4, n4 = first
    st = [(c4.view(G, T, d // 2), s4.view(G, T, d // g4), z4.view(G, T, d // g4),
           b4.view(G, T, m // 32), n4.view(G, T))]
    while len(st) < ncopies(R * per_tok):
        st.append(tuple(x.clone() for x in st[0]))
    gbs("residual_scores_f16_m256_g32", R * (per_tok + 4) + G * d * 2 + m * d * 2,
        [lambda a=a: K.scores_residual(q, S, *a, g4) for a in st])
    res["residual_scores_f16_m256_g32"]["scores/s"] = round(
        R / res["residual_scores_f16_m256_g32"]["ms"] * 1e3, 1)
    del kk, sk, b3, st, first
    torch.cuda.empty_cache()

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
    res["int8_round_trip_error"] = acc
    log(f"  int8_round_trip_error: {acc}")
    return res


def cpu_baseline(si, np, seconds):
    """The fp64 oracle's decode on one thread over whole groups of the same
    workload, until `seconds` of compute have been timed (at least 2)."""
    from threadpoolctl import threadpool_limits
    from oracle import decode as OD, int8 as OI, qjl as OQ
    W, B, H, T, d, m = si.W_DECODE, 16, 32, 32768, 128, 256
    S = si.projection(W, m, d, "f16")
    q = si.queries(W, B * H, 1, d, "f16")[:, 0]
    lam = 1.0 / math.sqrt(d)
    done, spent = 0, 0.0
    while done < B * H and (spent < seconds or done < 2):
        # group `done` is rows [done * T, (done + 1) * T) of the [B*H*T, d] tensors
        k = si.stream(W, si.K, T * d, "f16", start=done * T * d).reshape(T, d)
        v = si.stream(W, si.V, T * d, "f16", start=done * T * d).reshape(T, d)
        kw, kn = OQ.qjl_sketch(k, S)                  # cache build (untimed)
        vc, vs = OI.quantize_int8(v)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            OD.decode_qjl_int8(q[done:done + 1], S, kw[None], kn[None], vc[None], vs[None], lam)
            spent += time.perf_counter() - t0
        done += 1
    return {"value": round(done * T / spent, 1), "unit": "scores/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {B * H} (batch, head) groups x {T} tokens, one decode query each; "
                      f"fp64 numpy oracle on one thread, {spent:.1f} s of compute timed"}


def main():
    args = parse_args()
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

    comp = None
    if not args.no_components:
        del kbits, knorms, vcodes, vscales
        torch.cuda.empty_cache()
        log("bench: components")
        comp = components(K, si, torch, np)

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(si, np, args.cpu_seconds)

    line = {
        "metric": "KV quantize/dequant HBM GB/s (% of peak); QJL+INT8 decode scores/sec",
        "value": round(value, 1),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "graph_ms_per_step": round(graph_ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "decode step over a QJL-key / INT8-value cache: batch 16 x 32 heads "
                               "x 32768 tokens x d 128, m 256, 1 fp16 query per head, newest token "
                               "compressed in-step",
                   "global_batch": 16, "seq_len": T, "heads": H, "head_dim": d, "qjl_m": m,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "components": comp,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
