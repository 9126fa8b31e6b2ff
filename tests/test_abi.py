"""The C ABI on the CPU: the library loads, exports every function that
include/kvq.h declares, and rejects invalid arguments with a status and a
message before making any HIP call (so no GPU is needed here)."""
import ctypes
import os
import re
import subprocess

import pytest

from kv_cache_compression_kvq_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

A = 0x10000          # an aligned fake device address; never dereferenced
MIS = 0x10004        # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_functions()
    assert set(names) == set(L.PROTOTYPES), names


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r"\bT (kvq_[a-z0-9_]+)", out.stdout))
    assert set(declared_functions()) <= exported


def test_status_strings():
    lib = L.lib()
    names = ["KVQ_OK", "KVQ_ERR_NULL", "KVQ_ERR_SHAPE", "KVQ_ERR_ALIGN", "KVQ_ERR_DTYPE",
             "KVQ_ERR_WORKSPACE", "KVQ_ERR_LAUNCH"]
    for code, name in enumerate(names):
        assert lib.kvq_status_string(code).decode() == name
    assert lib.kvq_status_string(99).decode() == "KVQ_ERR_UNKNOWN"


def _err(status, expect):
    assert status == expect, (status, L.lib().kvq_last_error())
    assert L.lib().kvq_last_error().decode()


def test_quantize_validation():
    f = L.lib().kvq_quantize_int8
    _err(f(None, L.KVQ_F32, 4, 128, A, A, None), L.KVQ_ERR_NULL)
    _err(f(A, L.KVQ_F32, 4, 128, None, A, None), L.KVQ_ERR_NULL)
    _err(f(A, L.KVQ_F32, 4, 128, A, None, None), L.KVQ_ERR_NULL)
    _err(f(MIS, L.KVQ_F32, 4, 128, A, A, None), L.KVQ_ERR_ALIGN)
    _err(f(A, L.KVQ_F32, 4, 128, MIS, A, None), L.KVQ_ERR_ALIGN)
    _err(f(A, L.KVQ_F32, -1, 128, A, A, None), L.KVQ_ERR_SHAPE)
    for d in (0, 8, 120, 65552, -16):
        _err(f(A, L.KVQ_F32, 4, d, A, A, None), L.KVQ_ERR_SHAPE)
    _err(f(A, 7, 4, 128, A, A, None), L.KVQ_ERR_DTYPE)
    # zero rows is a no-op, even with NULL pointers
    assert f(None, L.KVQ_F32, 0, 128, None, None, None) == L.KVQ_OK


def test_dequantize_validation():
    f = L.lib().kvq_dequantize_int8
    _err(f(None, A, 4, 128, A, L.KVQ_F32, None), L.KVQ_ERR_NULL)
    _err(f(A, A, 4, 128, None, L.KVQ_F16, None), L.KVQ_ERR_NULL)
    _err(f(A, MIS, 4, 128, A, L.KVQ_F32, None), L.KVQ_ERR_ALIGN)
    _err(f(A, A, 4, 100, A, L.KVQ_F32, None), L.KVQ_ERR_SHAPE)
    _err(f(A, A, 4, 128, A, 2, None), L.KVQ_ERR_DTYPE)
    assert f(None, None, 0, 128, None, L.KVQ_F32, None) == L.KVQ_OK


def test_int4_validation():
    q = L.lib().kvq_quantize_int4
    _err(q(None, L.KVQ_F32, 4, 128, 32, A, A, A, None), L.KVQ_ERR_NULL)
    _err(q(A, L.KVQ_F32, 4, 128, 32, A, A, None, None), L.KVQ_ERR_NULL)
    _err(q(A, L.KVQ_F32, 4, 128, 32, A, MIS, A, None), L.KVQ_ERR_ALIGN)
    _err(q(A, L.KVQ_F32, -1, 128, 32, A, A, A, None), L.KVQ_ERR_SHAPE)
    for g in (0, 8, 24, 48, 256, -32):      # not a multiple of 16 dividing 128
        _err(q(A, L.KVQ_F32, 4, 128, g, A, A, A, None), L.KVQ_ERR_SHAPE)
    _err(q(A, L.KVQ_F32, 4, 100, 20, A, A, A, None), L.KVQ_ERR_SHAPE)
    _err(q(A, 2, 4, 128, 32, A, A, A, None), L.KVQ_ERR_DTYPE)
    assert q(None, L.KVQ_F16, 0, 96, 48, None, None, None, None) == L.KVQ_OK
    dq = L.lib().kvq_dequantize_int4
    _err(dq(A, A, None, 4, 128, 32, A, L.KVQ_F32, None), L.KVQ_ERR_NULL)
    _err(dq(A, A, A, 4, 128, 32, MIS, L.KVQ_F32, None), L.KVQ_ERR_ALIGN)
    _err(dq(A, A, A, 4, 128, 40, A, L.KVQ_F32, None), L.KVQ_ERR_SHAPE)
    _err(dq(A, A, A, 4, 128, 32, A, 3, None), L.KVQ_ERR_DTYPE)
    assert dq(None, None, None, 0, 128, 32, None, L.KVQ_F16, None) == L.KVQ_OK


def test_residual_sketch_validation():
    f = L.lib().kvq_residual_sketch
    ok = (A, L.KVQ_F16, 4, 128, 32, A, L.KVQ_F16, 256, A, A, A, A, A, None)

    def call(**kw):
        names = ["k", "k_dt", "rows", "d", "g", "S", "S_dt", "m", "codes", "steps", "offsets",
                 "bits", "norms", "stream"]
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])

    for name in ("k", "S", "codes", "steps", "offsets", "bits", "norms"):
        _err(call(**{name: None}), L.KVQ_ERR_NULL)
        _err(call(**{name: MIS}), L.KVQ_ERR_ALIGN)
    _err(call(rows=-1), L.KVQ_ERR_SHAPE)
    for d in (0, 8, 1040, 2048):
        _err(call(d=d, g=16), L.KVQ_ERR_SHAPE)
    for g in (0, 8, 48, 256):
        _err(call(g=g), L.KVQ_ERR_SHAPE)
    for m in (0, 16, 48, 2048):
        _err(call(m=m), L.KVQ_ERR_SHAPE)
    _err(call(k_dt=5), L.KVQ_ERR_DTYPE)
    _err(call(S_dt=-1), L.KVQ_ERR_DTYPE)
    assert f(None, L.KVQ_F16, 0, 128, 32, None, L.KVQ_F16, 256, None, None, None, None, None,
             None) == L.KVQ_OK


def test_scores_int8_validation():
    f = L.lib().kvq_scores_int8
    _err(f(A, L.KVQ_F16, 2, 0, A, A, 16, 128, A, None), L.KVQ_ERR_SHAPE)
    _err(f(A, L.KVQ_F16, 2, 65, A, A, 16, 128, A, None), L.KVQ_ERR_SHAPE)
    _err(f(A, L.KVQ_F16, -2, 1, A, A, 16, 128, A, None), L.KVQ_ERR_SHAPE)
    _err(f(A, L.KVQ_F16, 2, 1, A, A, -16, 128, A, None), L.KVQ_ERR_SHAPE)
    _err(f(A, L.KVQ_F16, 2, 1, A, A, 16, 128, None, None), L.KVQ_ERR_NULL)
    _err(f(A, 5, 2, 1, A, A, 16, 128, A, None), L.KVQ_ERR_DTYPE)
    assert f(None, L.KVQ_F16, 0, 1, None, None, 16, 128, None, None) == L.KVQ_OK
    assert f(None, L.KVQ_F16, 2, 1, None, None, 0, 128, None, None) == L.KVQ_OK


def test_sketch_validation():
    f = L.lib().kvq_qjl_sketch
    for m in (0, 16, 48, 1056, 2048):
        _err(f(A, L.KVQ_F16, 4, 128, A, m, A, A, None), L.KVQ_ERR_SHAPE)
    _err(f(A, L.KVQ_F16, 4, 128, None, 256, A, A, None), L.KVQ_ERR_NULL)
    _err(f(A, L.KVQ_F16, 4, 128, A, 256, A, MIS, None), L.KVQ_ERR_ALIGN)
    _err(f(A, 3, 4, 128, A, 256, A, A, None), L.KVQ_ERR_DTYPE)
    assert f(None, L.KVQ_F16, 0, 128, None, 256, None, None, None) == L.KVQ_OK


def test_scores_qjl_validation():
    f = L.lib().kvq_scores_qjl
    _err(f(A, L.KVQ_F16, 2, 1, A, L.KVQ_F16, 40, A, A, 16, 128, A, None), L.KVQ_ERR_SHAPE)
    _err(f(A, L.KVQ_F16, 2, 1, A, 9, 256, A, A, 16, 128, A, None), L.KVQ_ERR_DTYPE)
    _err(f(A, L.KVQ_F16, 2, 1, A, L.KVQ_F16, 256, None, A, 16, 128, A, None), L.KVQ_ERR_NULL)
    assert f(None, L.KVQ_F16, 2, 1, None, L.KVQ_F16, 256, None, None, 0, 128, None, None) == L.KVQ_OK


def test_decode_validation():
    f = L.lib().kvq_decode_qjl_int8
    args = [A, L.KVQ_F16, 2, A, L.KVQ_F16, 256, A, A, A, A, 16, 128, 0.1, A, 1 << 20, A, None]

    def call(**kw):
        a = list(args)
        names = ["q", "q_dt", "groups", "S", "S_dt", "m", "kbits", "knorms", "vcodes", "vscales",
                 "T", "d", "sm", "ws", "ws_bytes", "out", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    _err(call(T=0), L.KVQ_ERR_SHAPE)
    _err(call(m=33), L.KVQ_ERR_SHAPE)
    _err(call(d=24), L.KVQ_ERR_SHAPE)
    _err(call(vcodes=None), L.KVQ_ERR_NULL)
    _err(call(out=MIS), L.KVQ_ERR_ALIGN)
    _err(call(q_dt=4), L.KVQ_ERR_DTYPE)
    assert call(groups=0, q=None, S=None, kbits=None, knorms=None, vcodes=None, vscales=None,
                ws=None, out=None) == L.KVQ_OK


def test_decode_noalloc_validation():
    """The allocation-free decode validates like the workspace form (before any
    HIP call), and has no workspace argument to get wrong."""
    f = L.lib().kvq_decode_qjl_int8_noalloc
    args = [A, L.KVQ_F16, 2, A, L.KVQ_F16, 256, A, A, A, A, 16, 128, 0.1, A, None]
    names = ["q", "q_dt", "groups", "S", "S_dt", "m", "kbits", "knorms", "vcodes", "vscales",
             "T", "d", "sm", "out", "stream"]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    _err(call(T=0), L.KVQ_ERR_SHAPE)
    _err(call(m=33), L.KVQ_ERR_SHAPE)
    _err(call(d=24), L.KVQ_ERR_SHAPE)
    _err(call(d=2048), L.KVQ_ERR_SHAPE)
    _err(call(groups=-3), L.KVQ_ERR_SHAPE)
    _err(call(kbits=None), L.KVQ_ERR_NULL)
    _err(call(out=None), L.KVQ_ERR_NULL)
    _err(call(vscales=MIS), L.KVQ_ERR_ALIGN)
    _err(call(S_dt=3), L.KVQ_ERR_DTYPE)
    assert call(groups=0, q=None, S=None, kbits=None, knorms=None, vcodes=None, vscales=None,
                out=None) == L.KVQ_OK


def test_cache_append_validation():
    f = L.lib().kvq_cache_append
    args = [A, A, L.KVQ_F16, 4, 128, A, 256, 16, 15, A, A, A, A, None]
    names = ["k", "v", "dt", "groups", "d", "S", "m", "T", "pos", "kbits", "knorms", "vcodes",
             "vscales", "stream"]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    _err(call(pos=16), L.KVQ_ERR_SHAPE)
    _err(call(pos=-1), L.KVQ_ERR_SHAPE)
    _err(call(T=0), L.KVQ_ERR_SHAPE)
    _err(call(d=2048), L.KVQ_ERR_SHAPE)
    _err(call(d=120), L.KVQ_ERR_SHAPE)
    _err(call(m=48), L.KVQ_ERR_SHAPE)
    _err(call(groups=-1), L.KVQ_ERR_SHAPE)
    _err(call(dt=2), L.KVQ_ERR_DTYPE)
    _err(call(v=None), L.KVQ_ERR_NULL)
    _err(call(kbits=None), L.KVQ_ERR_NULL)
    _err(call(vscales=MIS), L.KVQ_ERR_ALIGN)
    assert call(groups=0, k=None, v=None, S=None, kbits=None, knorms=None, vcodes=None,
                vscales=None) == L.KVQ_OK


def test_workspace_query_rejects_bad_shapes_without_a_device():
    f = L.lib().kvq_decode_workspace_bytes
    assert f(0, 16, 128, 256) == 0
    assert f(4, 0, 128, 256) == 0
    assert f(4, 16, 100, 256) == 0
    assert f(4, 16, 128, 48) == 0
    assert f(4, 16, 2048, 256) == 0


def test_python_binding_requires_gpu_tensors():
    import torch
    from kv_cache_compression_kvq_amd import ops
    with pytest.raises(ValueError, match="GPU tensor"):
        ops.quantize_int8(torch.zeros(4, 128))


def test_scores_residual_validation():
    f = L.lib().kvq_scores_residual
    names = ["q", "q_dt", "groups", "nq", "S", "S_dt", "m", "g", "codes", "steps", "offsets",
             "bits", "norms", "T", "d", "scores", "stream"]
    ok = (A, L.KVQ_F16, 2, 1, A, L.KVQ_F16, 256, 32, A, A, A, A, A, 16, 128, A, None)

    def call(**kw):
        args = dict(zip(names, ok))
        args.update(kw)
        return f(*[args[n] for n in names])

    for name in ("q", "S", "codes", "steps", "offsets", "bits", "norms", "scores"):
        _err(call(**{name: None}), L.KVQ_ERR_NULL)
        _err(call(**{name: MIS}), L.KVQ_ERR_ALIGN)
    for kw in ({"groups": -1}, {"T": -1}, {"nq": 0}, {"nq": 65}, {"d": 2048, "g": 128},
               {"g": 24}, {"m": 48}):
        _err(call(**kw), L.KVQ_ERR_SHAPE)
    _err(call(q_dt=3), L.KVQ_ERR_DTYPE)
    assert call(groups=0, q=None, S=None, codes=None, steps=None, offsets=None, bits=None,
                norms=None, scores=None) == L.KVQ_OK
    assert call(T=0, scores=None) == L.KVQ_OK


def test_int8_channel_validation():
    qf = L.lib().kvq_quantize_int8_channel
    _err(qf(None, L.KVQ_F16, 2, 64, 128, A, A, None), L.KVQ_ERR_NULL)
    _err(qf(A, L.KVQ_F16, 2, 64, 128, MIS, A, None), L.KVQ_ERR_ALIGN)
    for d in (0, 8, 8208, 100):
        _err(qf(A, L.KVQ_F16, 2, 64, d, A, A, None), L.KVQ_ERR_SHAPE)
    _err(qf(A, L.KVQ_F16, -1, 64, 128, A, A, None), L.KVQ_ERR_SHAPE)
    _err(qf(A, L.KVQ_F16, 2, -64, 128, A, A, None), L.KVQ_ERR_SHAPE)
    _err(qf(A, 9, 2, 64, 128, A, A, None), L.KVQ_ERR_DTYPE)
    assert qf(None, L.KVQ_F16, 0, 64, 128, None, None, None) == L.KVQ_OK
    assert qf(None, L.KVQ_F16, 2, 0, 128, None, None, None) == L.KVQ_OK
    dq = L.lib().kvq_dequantize_int8_channel
    _err(dq(A, None, 2, 64, 128, A, L.KVQ_F32, None), L.KVQ_ERR_NULL)
    _err(dq(A, A, 2, 64, 120, A, L.KVQ_F32, None), L.KVQ_ERR_SHAPE)
    _err(dq(A, A, 2, 64, 128, A, 4, None), L.KVQ_ERR_DTYPE)
    sc = L.lib().kvq_scores_int8_channel
    _err(sc(A, L.KVQ_F16, 2, 0, A, A, 64, 128, A, None), L.KVQ_ERR_SHAPE)
    _err(sc(A, L.KVQ_F16, 2, 1, A, A, 64, 16384, A, None), L.KVQ_ERR_SHAPE)
    _err(sc(A, L.KVQ_F16, 2, 1, A, MIS, 64, 128, A, None), L.KVQ_ERR_ALIGN)
    assert sc(None, L.KVQ_F16, 2, 1, None, None, 0, 128, None, None) == L.KVQ_OK


def test_decode_gqa_validation():
    f = L.lib().kvq_decode_qjl_int8_gqa
    args = [A, L.KVQ_F16, 2, 4, A, L.KVQ_F16, 256, A, A, A, A, 16, 128, 0.1, A, 1 << 20, A, None]
    names = ["q", "q_dt", "groups", "nq", "S", "S_dt", "m", "kbits", "knorms", "vcodes", "vscales",
             "T", "d", "sm", "ws", "ws_bytes", "out", "stream"]

    def call(**kw):
        a = list(args)
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    _err(call(nq=0), L.KVQ_ERR_SHAPE)
    _err(call(nq=65), L.KVQ_ERR_SHAPE)
    _err(call(T=0), L.KVQ_ERR_SHAPE)
    _err(call(out=None), L.KVQ_ERR_NULL)
    _err(call(q=MIS), L.KVQ_ERR_ALIGN)
    _err(call(S_dt=7), L.KVQ_ERR_DTYPE)
    assert call(groups=0, q=None, S=None, kbits=None, knorms=None, vcodes=None, vscales=None,
                ws=None, out=None) == L.KVQ_OK
    assert L.lib().kvq_decode_gqa_workspace_bytes(2, 0, 16, 128, 256) == 0
    assert L.lib().kvq_decode_gqa_workspace_bytes(2, 4, 16, 120, 256) == 0
