"""Torch-facing wrappers of the libkvq C ABI.

Argument marshalling only: dtype/device/contiguity checks, output allocation
with torch, and the current HIP stream.  Every step of the computation runs
in libkvq's kernels.  Sign words are returned as int32 tensors (the bytes of
the ABI's uint32 words); norms as float16 tensors (the ABI's binary16 bits).
"""
from __future__ import annotations

import math

import torch

from . import _lib as L

_DT = {torch.float32: L.KVQ_F32, torch.float16: L.KVQ_F16}


def _dtype_code(t: torch.Tensor, what: str) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"{what}: expected float32 or float16, got {t.dtype}") from None


def _dev(t: torch.Tensor, what: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{what} must be a GPU tensor (libkvq has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _p(t: torch.Tensor):
    return t.data_ptr() if t.numel() else None


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _out(given, shape, dtype, like: torch.Tensor, what: str) -> torch.Tensor:
    """The caller's output tensor (checked: shape, dtype, device, contiguous)
    or a new one; passing outputs makes a call allocation-free."""
    shape = tuple(shape)
    if given is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if tuple(given.shape) != shape or given.dtype != dtype or given.device != like.device:
        raise ValueError(f"{what}: expected {dtype} {shape} on {like.device}, got "
                         f"{given.dtype} {tuple(given.shape)} on {given.device}")
    return _dev(given, what)


def quantize_int8(x: torch.Tensor, out=None) -> tuple[torch.Tensor, torch.Tensor]:
    """x [..., d] fp32/fp16 -> (codes int8 [..., d], scales fp32 [...]).
    ``out``: optional (codes, scales) to write into."""
    _dev(x, "x")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    codes = _out(out and out[0], x.shape, torch.int8, x, "codes")
    scales = _out(out and out[1], x.shape[:-1], torch.float32, x, "scales")
    L.check(L.lib().kvq_quantize_int8(_p(x), _dtype_code(x, "x"), rows, d, _p(codes),
                                      _p(scales), _stream(x)))
    return codes, scales


def dequantize_int8(codes: torch.Tensor, scales: torch.Tensor,
                    out_dtype: torch.dtype = torch.float32, out=None) -> torch.Tensor:
    """codes int8 [..., d], scales fp32 [...] -> [..., d] in out_dtype."""
    _dev(codes, "codes"), _dev(scales, "scales")
    if codes.dtype != torch.int8 or scales.dtype != torch.float32:
        raise TypeError("codes must be int8 and scales float32")
    d = codes.shape[-1]
    rows = codes.numel() // d if d else 0
    if scales.numel() != rows:
        raise ValueError(f"scales has {scales.numel()} entries for {rows} rows")
    out = _out(out, codes.shape, out_dtype, codes, "out")
    L.check(L.lib().kvq_dequantize_int8(_p(codes), _p(scales), rows, d, _p(out),
                                        _dtype_code(out, "out_dtype"), _stream(codes)))
    return out


def quantize_int8_channel(x: torch.Tensor, out=None) -> tuple[torch.Tensor, torch.Tensor]:
    """Keys x [G, T, d] fp32/fp16 -> (codes int8 [G, T, d], per-channel
    scales fp32 [G, d]).  ``out``: optional (codes, scales)."""
    _dev(x, "x")
    G, T, d = x.shape
    codes = _out(out and out[0], (G, T, d), torch.int8, x, "codes")
    scales = _out(out and out[1], (G, d), torch.float32, x, "scales")
    L.check(L.lib().kvq_quantize_int8_channel(_p(x), _dtype_code(x, "x"), G, T, d, _p(codes),
                                              _p(scales), _stream(x)))
    return codes, scales


def dequantize_int8_channel(codes: torch.Tensor, scales: torch.Tensor,
                            out_dtype: torch.dtype = torch.float32, out=None) -> torch.Tensor:
    """codes int8 [G, T, d], scales fp32 [G, d] -> [G, T, d] in out_dtype."""
    _dev(codes, "codes"), _dev(scales, "scales")
    if codes.dtype != torch.int8 or scales.dtype != torch.float32:
        raise TypeError("codes must be int8 and scales float32")
    G, T, d = codes.shape
    if tuple(scales.shape) != (G, d):
        raise ValueError(f"scales {tuple(scales.shape)} for codes {tuple(codes.shape)}")
    out = _out(out, (G, T, d), out_dtype, codes, "out")
    L.check(L.lib().kvq_dequantize_int8_channel(_p(codes), _p(scales), G, T, d, _p(out),
                                                _dtype_code(out, "out_dtype"), _stream(codes)))
    return out


def scores_int8_channel(q: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                        out=None) -> torch.Tensor:
    """q [G, nq, d]; codes [G, T, d] int8; scales [G, d] -> scores [G, nq, T] fp32."""
    _dev(q, "q"), _dev(codes, "codes"), _dev(scales, "scales")
    G, nq, d = q.shape
    if codes.shape[0] != G or codes.shape[2] != d or tuple(scales.shape) != (G, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, codes {tuple(codes.shape)}, "
                         f"scales {tuple(scales.shape)}")
    T = codes.shape[1]
    out = _out(out, (G, nq, T), torch.float32, q, "out")
    L.check(L.lib().kvq_scores_int8_channel(_p(q), _dtype_code(q, "q"), G, nq, _p(codes),
                                            _p(scales), T, d, _p(out), _stream(q)))
    return out


def quantize_int4(x: torch.Tensor, g: int,
                  out=None) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """x [..., d] fp32/fp16, group size g -> (codes uint8 [..., d/2] two per
    byte, steps fp32 [..., d/g], offsets fp32 [..., d/g]).  ``out``: optional
    (codes, steps, offsets)."""
    _dev(x, "x")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    ng = d // g if g > 0 else 0
    codes = _out(out and out[0], (*x.shape[:-1], d // 2), torch.uint8, x, "codes")
    steps = _out(out and out[1], (*x.shape[:-1], ng), torch.float32, x, "steps")
    offsets = _out(out and out[2], (*x.shape[:-1], ng), torch.float32, x, "offsets")
    L.check(L.lib().kvq_quantize_int4(_p(x), _dtype_code(x, "x"), rows, d, g, _p(codes), _p(steps),
                                      _p(offsets), _stream(x)))
    return codes, steps, offsets


def dequantize_int4(codes: torch.Tensor, steps: torch.Tensor, offsets: torch.Tensor, g: int,
                    out_dtype: torch.dtype = torch.float32, out=None) -> torch.Tensor:
    """codes uint8 [..., d/2], steps / offsets fp32 [..., d/g] -> [..., d]."""
    _dev(codes, "codes"), _dev(steps, "steps"), _dev(offsets, "offsets")
    if codes.dtype != torch.uint8 or steps.dtype != torch.float32 or offsets.dtype != torch.float32:
        raise TypeError("codes must be uint8, steps and offsets float32")
    d = 2 * codes.shape[-1]
    rows = codes.numel() * 2 // d if d else 0
    if g <= 0 or d % g != 0 or steps.shape != offsets.shape or steps.numel() != rows * (d // g):
        raise ValueError(f"shape mismatch: codes {tuple(codes.shape)}, g {g}, "
                         f"steps {tuple(steps.shape)}, offsets {tuple(offsets.shape)}")
    out = _out(out, (*codes.shape[:-1], d), out_dtype, codes, "out")
    L.check(L.lib().kvq_dequantize_int4(_p(codes), _p(steps), _p(offsets), rows, d, g, _p(out),
                                        _dtype_code(out, "out_dtype"), _stream(codes)))
    return out


def scores_int8(q: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                out=None) -> torch.Tensor:
    """q [G, nq, d]; codes [G, T, d] int8; scales [G, T] -> scores [G, nq, T] fp32."""
    _dev(q, "q"), _dev(codes, "codes"), _dev(scales, "scales")
    G, nq, d = q.shape
    if codes.shape[0] != G or codes.shape[2] != d or tuple(scales.shape) != tuple(codes.shape[:2]):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, codes {tuple(codes.shape)}, "
                         f"scales {tuple(scales.shape)}")
    T = codes.shape[1]
    out = _out(out, (G, nq, T), torch.float32, q, "out")
    L.check(L.lib().kvq_scores_int8(_p(q), _dtype_code(q, "q"), G, nq, _p(codes), _p(scales), T, d,
                                    _p(out), _stream(q)))
    return out


def qjl_sketch(k: torch.Tensor, S: torch.Tensor, out=None) -> tuple[torch.Tensor, torch.Tensor]:
    """k [..., d] and S [m, d] of the same dtype -> (sign words int32 [..., m // 32],
    norms fp16 [...]).  ``out``: optional (bits, norms)."""
    _dev(k, "k"), _dev(S, "S")
    if S.dtype != k.dtype:
        raise TypeError("S must have the keys' dtype")
    m, d = S.shape
    if k.shape[-1] != d:
        raise ValueError(f"k has d = {k.shape[-1]}, S has d = {d}")
    rows = k.numel() // d if d else 0
    bits = _out(out and out[0], (*k.shape[:-1], m // 32), torch.int32, k, "bits")
    norms = _out(out and out[1], k.shape[:-1], torch.float16, k, "norms")
    L.check(L.lib().kvq_qjl_sketch(_p(k), _dtype_code(k, "k"), rows, d, _p(S), m, _p(bits),
                                   _p(norms), _stream(k)))
    return bits, norms


def residual_sketch(k: torch.Tensor, S: torch.Tensor, g: int, out=None):
    """Two-stage key compression: k [..., d] fp32/fp16, S [m, d] fp32/fp16,
    group size g -> (codes uint8 [..., d/2], steps fp32 [..., d/g],
    offsets fp32 [..., d/g], residual sign words int32 [..., m // 32],
    residual norms fp16 [...]).  ``out``: optional tuple of the five outputs."""
    _dev(k, "k"), _dev(S, "S")
    m, d = S.shape
    if k.shape[-1] != d:
        raise ValueError(f"k has d = {k.shape[-1]}, S has d = {d}")
    rows = k.numel() // d if d else 0
    lead = k.shape[:-1]
    ng = d // g if g > 0 else 0
    o = out or (None,) * 5
    codes = _out(o[0], (*lead, d // 2), torch.uint8, k, "codes")
    steps = _out(o[1], (*lead, ng), torch.float32, k, "steps")
    offsets = _out(o[2], (*lead, ng), torch.float32, k, "offsets")
    bits = _out(o[3], (*lead, m // 32), torch.int32, k, "bits")
    norms = _out(o[4], lead, torch.float16, k, "norms")
    L.check(L.lib().kvq_residual_sketch(_p(k), _dtype_code(k, "k"), rows, d, g, _p(S),
                                        _dtype_code(S, "S"), m, _p(codes), _p(steps), _p(offsets),
                                        _p(bits), _p(norms), _stream(k)))
    return codes, steps, offsets, bits, norms


def scores_residual(q: torch.Tensor, S: torch.Tensor, codes: torch.Tensor, steps: torch.Tensor,
                    offsets: torch.Tensor, bits: torch.Tensor, norms: torch.Tensor,
                    g: int, out=None) -> torch.Tensor:
    """q [G, nq, d]; S [m, d]; codes [G, T, d/2]; steps / offsets [G, T, d/g];
    bits [G, T, m // 32]; norms [G, T] -> scores [G, nq, T] fp32."""
    for t, n in ((q, "q"), (S, "S"), (codes, "codes"), (steps, "steps"), (offsets, "offsets"),
                 (bits, "bits"), (norms, "norms")):
        _dev(t, n)
    G, nq, d = q.shape
    m = S.shape[0]
    T = codes.shape[1]
    ng = d // g if g > 0 else 0
    if (S.shape[1] != d or codes.shape != (G, T, d // 2) or steps.shape != (G, T, ng)
            or offsets.shape != (G, T, ng) or bits.shape != (G, T, m // 32) or norms.shape != (G, T)):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, S {tuple(S.shape)}, codes "
                         f"{tuple(codes.shape)}, steps {tuple(steps.shape)}, bits {tuple(bits.shape)}, "
                         f"norms {tuple(norms.shape)}, g {g}")
    out = _out(out, (G, nq, T), torch.float32, q, "out")
    L.check(L.lib().kvq_scores_residual(_p(q), _dtype_code(q, "q"), G, nq, _p(S), _dtype_code(S, "S"),
                                        m, g, _p(codes), _p(steps), _p(offsets), _p(bits), _p(norms),
                                        T, d, _p(out), _stream(q)))
    return out


def scores_qjl(q: torch.Tensor, S: torch.Tensor, bits: torch.Tensor,
               norms: torch.Tensor, out=None) -> torch.Tensor:
    """q [G, nq, d]; S [m, d]; bits [G, T, m // 32]; norms [G, T] -> [G, nq, T] fp32."""
    for t, n in ((q, "q"), (S, "S"), (bits, "bits"), (norms, "norms")):
        _dev(t, n)
    G, nq, d = q.shape
    m = S.shape[0]
    T = bits.shape[1]
    if bits.shape != (G, T, m // 32) or norms.shape != (G, T) or S.shape[1] != d:
        raise ValueError("shape mismatch between q, S, bits and norms")
    out = _out(out, (G, nq, T), torch.float32, q, "out")
    L.check(L.lib().kvq_scores_qjl(_p(q), _dtype_code(q, "q"), G, nq, _p(S), _dtype_code(S, "S"), m,
                                   _p(bits), _p(norms), T, d, _p(out), _stream(q)))
    return out


def decode_workspace_bytes(groups: int, T: int, d: int, m: int) -> int:
    return int(L.lib().kvq_decode_workspace_bytes(groups, T, d, m))


def decode_gqa_workspace_bytes(groups: int, nq: int, T: int, d: int, m: int) -> int:
    return int(L.lib().kvq_decode_gqa_workspace_bytes(groups, nq, T, d, m))


def decode_qjl_int8_gqa(q: torch.Tensor, S: torch.Tensor, kbits: torch.Tensor,
                        knorms: torch.Tensor, vcodes: torch.Tensor, vscales: torch.Tensor,
                        sm_scale: float | None = None, workspace: torch.Tensor | None = None,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step for grouped-query attention: q [G, nq, d] (nq query
    heads per KV head) against the group's QJL keys and INT8 values.
    Returns out [G, nq, d] fp32."""
    for t, n in ((q, "q"), (S, "S"), (kbits, "kbits"), (knorms, "knorms"), (vcodes, "vcodes"),
                 (vscales, "vscales")):
        _dev(t, n)
    G, nq, d = q.shape
    m = S.shape[0]
    T = kbits.shape[1]
    if (kbits.shape != (G, T, m // 32) or knorms.shape != (G, T) or vcodes.shape != (G, T, d)
            or vscales.shape != (G, T) or S.shape[1] != d):
        raise ValueError("shape mismatch between q, S and the cache tensors")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    need = decode_gqa_workspace_bytes(G, nq, T, d, m)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    out = _out(out, (G, nq, d), torch.float32, q, "out")
    L.check(L.lib().kvq_decode_qjl_int8_gqa(
        _p(q), _dtype_code(q, "q"), G, nq, _p(S), _dtype_code(S, "S"), m, _p(kbits), _p(knorms),
        _p(vcodes), _p(vscales), T, d, float(sm_scale), _p(workspace), workspace.numel(), _p(out),
        _stream(q)))
    return out


def decode_qjl_int8(q: torch.Tensor, S: torch.Tensor, kbits: torch.Tensor, knorms: torch.Tensor,
                    vcodes: torch.Tensor, vscales: torch.Tensor, sm_scale: float | None = None,
                    workspace: torch.Tensor | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """One decode step: q [G, d] against QJL keys (kbits [G, T, m // 32],
    knorms [G, T]) and INT8 values (vcodes [G, T, d], vscales [G, T]).
    Returns out [G, d] fp32.  ``workspace`` (uint8, >= decode_workspace_bytes)
    and ``out`` may be passed to avoid allocations."""
    for t, n in ((q, "q"), (S, "S"), (kbits, "kbits"), (knorms, "knorms"), (vcodes, "vcodes"),
                 (vscales, "vscales")):
        _dev(t, n)
    G, d = q.shape
    m = S.shape[0]
    T = kbits.shape[1]
    if (kbits.shape != (G, T, m // 32) or knorms.shape != (G, T) or vcodes.shape != (G, T, d)
            or vscales.shape != (G, T) or S.shape[1] != d):
        raise ValueError("shape mismatch between q, S and the cache tensors")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(G, T, d, m)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    out = _out(out, (G, d), torch.float32, q, "out")
    L.check(L.lib().kvq_decode_qjl_int8(
        _p(q), _dtype_code(q, "q"), G, _p(S), _dtype_code(S, "S"), m, _p(kbits), _p(knorms),
        _p(vcodes), _p(vscales), T, d, float(sm_scale), _p(workspace), workspace.numel(), _p(out),
        _stream(q)))
    return out


def decode_qjl_int8_noalloc(q: torch.Tensor, S: torch.Tensor, kbits: torch.Tensor,
                            knorms: torch.Tensor, vcodes: torch.Tensor, vscales: torch.Tensor,
                            sm_scale: float | None = None,
                            out: torch.Tensor | None = None) -> torch.Tensor:
    """decode_qjl_int8 through the entry point that takes no workspace and
    allocates nothing (its scratch is a fixed per-device array inside the
    library).  Pass ``out`` [G, d] fp32 to make the whole call allocation-free."""
    for t, n in ((q, "q"), (S, "S"), (kbits, "kbits"), (knorms, "knorms"), (vcodes, "vcodes"),
                 (vscales, "vscales")):
        _dev(t, n)
    G, d = q.shape
    m = S.shape[0]
    T = kbits.shape[1]
    if (kbits.shape != (G, T, m // 32) or knorms.shape != (G, T) or vcodes.shape != (G, T, d)
            or vscales.shape != (G, T) or S.shape[1] != d):
        raise ValueError("shape mismatch between q, S and the cache tensors")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    out = _out(out, (G, d), torch.float32, q, "out")
    L.check(L.lib().kvq_decode_qjl_int8_noalloc(
        _p(q), _dtype_code(q, "q"), G, _p(S), _dtype_code(S, "S"), m, _p(kbits), _p(knorms),
        _p(vcodes), _p(vscales), T, d, float(sm_scale), _p(out), _stream(q)))
    return out


def cache_append(k: torch.Tensor, v: torch.Tensor, S: torch.Tensor, kbits: torch.Tensor,
                 knorms: torch.Tensor, vcodes: torch.Tensor, vscales: torch.Tensor,
                 pos: int) -> None:
    """Compress the newest key k [G, d] and value v [G, d] of every group into
    token position ``pos`` of the cache (kbits [G, T, m // 32], knorms [G, T],
    vcodes [G, T, d], vscales [G, T]), in place."""
    for t, n in ((k, "k"), (v, "v"), (S, "S"), (kbits, "kbits"), (knorms, "knorms"),
                 (vcodes, "vcodes"), (vscales, "vscales")):
        _dev(t, n)
    if v.dtype != k.dtype or S.dtype != k.dtype:
        raise TypeError("k, v and S must have one dtype")
    G, d = k.shape
    m = S.shape[0]
    T = kbits.shape[1] if kbits.dim() == 3 else 0
    if (v.shape != (G, d) or S.shape[1] != d or kbits.shape != (G, T, m // 32)
            or knorms.shape != (G, T) or vcodes.shape != (G, T, d) or vscales.shape != (G, T)):
        raise ValueError("shape mismatch between k, v, S and the cache tensors")
    if (kbits.dtype != torch.int32 or knorms.dtype != torch.float16 or vcodes.dtype != torch.int8
            or vscales.dtype != torch.float32):
        raise TypeError("cache dtypes: kbits int32, knorms float16, vcodes int8, vscales float32")
    L.check(L.lib().kvq_cache_append(_p(k), _p(v), _dtype_code(k, "k"), G, d, _p(S), m, T,
                                     int(pos), _p(kbits), _p(knorms), _p(vcodes), _p(vscales),
                                     _stream(k)))
