"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/pa.h declares, and rejects bad arguments before touching the device.

None of these calls launches work: each either fails validation or is an empty
batch, both of which return before any HIP API call.
"""
import ctypes
import os
import re

import pytest

import paged_kv_cache_463_amd as P
from paged_kv_cache_463_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

OK, NULL, DTYPE, SHAPE, UNSUP, WS, HIP, ALIGN = range(8)
FAKE = 0x7F0000000000          # 16-byte aligned stand-in address, never dereferenced
MIS = FAKE + 8                 # misaligned stand-in


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"PA_API\s+[\w\s\*]+?\b(pa_\w+)\s*\(", text)))


def test_header_declares_the_five_calls():
    syms = declared_symbols()
    for s in ("pa_reshape_and_cache", "pa_decode", "pa_decode_splitkv",
              "pa_decode_splitkv_workspace_bytes", "pa_prefill_chunked", "pa_status_string"):
        assert s in syms


def test_library_exports_every_declared_symbol():
    lib = P.lib()
    for s in declared_symbols():
        assert hasattr(lib, s), s
    assert set(declared_symbols()) == set(B.SIGNATURES)


def test_status_strings_and_version():
    lib = P.lib()
    assert lib.pa_version() >= 100
    for code in range(8):
        assert lib.pa_status_string(code).decode().startswith(B.STATUS_NAMES[code])
    assert b"unknown" in lib.pa_status_string(99)


def _decode(**kw):
    a = dict(out=FAKE, query=FAKE, k=FAKE, v=FAKE, block_stride=16 * 4 * 64, num_blocks=32, bt=FAKE,
             bt_stride=3, lens=FAKE, B=4, hq=4, hkv=4, d=64, bs=16, scale=0.125, dtype=0)
    a.update(kw)
    return P.lib().pa_decode(a["out"], a["query"], a["k"], a["v"], a["block_stride"], a["num_blocks"],
                             a["bt"], a["bt_stride"], a["lens"], a["B"], a["hq"], a["hkv"], a["d"],
                             a["bs"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), NULL), (dict(query=None), NULL), (dict(k=None), NULL), (dict(bt=None), NULL),
    (dict(lens=None), NULL), (dict(dtype=3), DTYPE), (dict(dtype=-1), DTYPE), (dict(bs=32), UNSUP),
    (dict(d=96), UNSUP), (dict(hq=6, hkv=4), SHAPE), (dict(hq=64, hkv=4), UNSUP),
    (dict(block_stride=100), SHAPE), (dict(B=-1), SHAPE), (dict(num_blocks=0), SHAPE),
    (dict(out=MIS), ALIGN), (dict(k=MIS), ALIGN), (dict(B=0), OK), (dict(B=0, out=None), OK),
])
def test_decode_argument_checks(kw, code):
    assert _decode(**kw) == code


def _scatter(**kw):
    a = dict(key=FAKE, value=FAKE, ts=8 * 128, k=FAKE, v=FAKE, bstride=16 * 8 * 128, nb=10, slots=FAKE,
             T=5, hkv=8, d=128, bs=16, dtype=2)
    a.update(kw)
    return P.lib().pa_reshape_and_cache(a["key"], a["value"], a["ts"], a["k"], a["v"], a["bstride"],
                                        a["nb"], a["slots"], a["T"], a["hkv"], a["d"], a["bs"],
                                        a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(key=None), NULL), (dict(slots=None), NULL), (dict(dtype=7), DTYPE), (dict(bs=8), UNSUP),
    (dict(ts=100), SHAPE), (dict(bstride=16), SHAPE), (dict(T=-3), SHAPE), (dict(ts=8 * 128 + 4), ALIGN),
    (dict(value=MIS), ALIGN), (dict(T=0, slots=None), OK),
])
def test_scatter_argument_checks(kw, code):
    assert _scatter(**kw) == code


def test_splitkv_workspace_and_checks():
    lib = P.lib()
    ws = lib.pa_decode_splitkv_workspace_bytes(8, 64, 128, 131072, 512)
    rows = 8 * 64 * 256
    assert ws >= rows * (128 + 2) * 4
    assert lib.pa_decode_splitkv_workspace_bytes(0, 64, 128, 100, 512) == 0

    def call(part=512, ws_ptr=FAKE, ws_bytes=ws, B=8, mcl=131072):
        return lib.pa_decode_splitkv(FAKE, FAKE, FAKE, FAKE, 16 * 8 * 128, 50000, FAKE, 8192, FAKE, B, 64, 8,
                                     128, 16, 0.088, 2, mcl, part, ws_ptr, ws_bytes, None)
    assert call(part=500) == SHAPE
    assert call(part=0) == SHAPE
    assert call(ws_bytes=ws - 1) == WS
    assert call(ws_ptr=None) == WS
    assert call(ws_ptr=MIS) == ALIGN
    assert call(B=0) == OK


def test_prefill_checks():
    lib = P.lib()

    def call(dtype=2, causal=1, cu=FAKE, T=8192, qmax=512, B=16):
        return lib.pa_prefill_chunked(FAKE, FAKE, cu, qmax, T, FAKE, FAKE, 16 * 8 * 128, 2816, FAKE, 160,
                                      FAKE, B, 32, 8, 128, 16, 0.088, causal, dtype, None)
    assert call(dtype=0) == DTYPE
    assert call(causal=2) == SHAPE
    assert call(cu=None) == NULL
    assert call(T=0) == OK
    assert call(B=0) == OK


def test_prefill_fp8_checks():
    lib = P.lib()

    def call(dtype=2, causal=1, cu=FAKE, T=8192, B=16, ks=FAKE, vs=FAKE, bstride=16 * 8 * 128):
        return lib.pa_prefill_chunked_fp8(FAKE, FAKE, cu, 512, T, FAKE, FAKE, bstride, 2816, FAKE, 160,
                                          FAKE, B, 32, 8, 128, 16, 0.088, causal, ks, vs, dtype, None)
    assert call(dtype=0) == DTYPE                  # fp32 queries are not read with an FP8 cache
    assert call(dtype=3) == DTYPE
    assert call(causal=2) == SHAPE
    assert call(cu=None) == NULL
    assert call(ks=None) == NULL and call(vs=None) == NULL
    assert call(bstride=16 * 8 * 128 - 1) == SHAPE  # one byte per element: at least 16 * H_kv * D
    assert call(bstride=16 * 8 * 128 + 8) == ALIGN
    assert call(T=0) == OK
    assert call(B=0) == OK


def _scatter_fp8(**kw):
    a = dict(key=FAKE, value=FAKE, ts=8 * 128, k=FAKE, v=FAKE, bstride=16 * 8 * 128, nb=10, slots=FAKE,
             T=5, hkv=8, d=128, bs=16, ks=FAKE, vs=FAKE, dtype=2)
    a.update(kw)
    return P.lib().pa_reshape_and_cache_fp8(a["key"], a["value"], a["ts"], a["k"], a["v"], a["bstride"],
                                            a["nb"], a["slots"], a["T"], a["hkv"], a["d"], a["bs"],
                                            a["ks"], a["vs"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ks=None), NULL), (dict(vs=None), NULL), (dict(key=None), NULL), (dict(dtype=3), DTYPE),
    (dict(d=96), UNSUP), (dict(bstride=16 * 8 * 128 - 16), SHAPE), (dict(bstride=16 * 8 * 128 + 8), ALIGN),
    (dict(ts=8 * 128 + 4), ALIGN), (dict(dtype=0, ts=8 * 128 + 2), ALIGN), (dict(T=0, ks=None), OK),
])
def test_scatter_fp8_argument_checks(kw, code):
    assert _scatter_fp8(**kw) == code


def _decode_fp8(split=False, **kw):
    a = dict(out=FAKE, query=FAKE, k=FAKE, v=FAKE, block_stride=16 * 4 * 128, num_blocks=32, bt=FAKE,
             bt_stride=3, lens=FAKE, B=4, hq=8, hkv=4, d=128, bs=16, scale=0.088, ks=FAKE, vs=FAKE, dtype=2,
             mcl=48, part=512, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    args = [a["out"], a["query"], a["k"], a["v"], a["block_stride"], a["num_blocks"], a["bt"], a["bt_stride"],
            a["lens"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["scale"], a["ks"], a["vs"], a["dtype"]]
    if split:
        return P.lib().pa_decode_splitkv_fp8(*args, a["mcl"], a["part"], a["ws"], a["wsb"], None)
    return P.lib().pa_decode_fp8(*args, None)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), DTYPE), (dict(dtype=3), DTYPE), (dict(ks=None), NULL), (dict(vs=None), NULL),
    (dict(out=None), NULL), (dict(d=96), UNSUP), (dict(hq=64, hkv=4), UNSUP),
    (dict(block_stride=16 * 4 * 128 - 16), SHAPE), (dict(block_stride=16 * 4 * 128 + 8), ALIGN),
    (dict(k=MIS), ALIGN), (dict(B=0), OK), (dict(B=0, ks=None), OK),
])
def test_decode_fp8_argument_checks(split, kw, code):
    assert _decode_fp8(split, **kw) == code


def test_splitkv_fp8_workspace_checks():
    assert _decode_fp8(True, wsb=16) == WS
    assert _decode_fp8(True, ws=None) == WS
    assert _decode_fp8(True, part=100) == SHAPE


def _step(fp8=False, **kw):
    a = dict(out=FAKE, query=FAKE, kn=FAKE, vn=FAKE, ts=4 * 128, k=FAKE, v=FAKE, block_stride=16 * 4 * 128,
             num_blocks=32, bt=FAKE, bt_stride=3, lens=FAKE, B=4, hq=8, hkv=4, d=128, bs=16, scale=0.088,
             ks=FAKE, vs=FAKE, dtype=2)
    a.update(kw)
    head = [a["out"], a["query"], a["kn"], a["vn"], a["ts"], a["k"], a["v"], a["block_stride"], a["num_blocks"],
            a["bt"], a["bt_stride"], a["lens"], a["B"], a["hq"], a["hkv"], a["d"], a["bs"], a["scale"]]
    if fp8:
        return P.lib().pa_decode_step_fp8(*head, a["ks"], a["vs"], a["dtype"], None)
    return P.lib().pa_decode_step(*head, a["dtype"], None)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), NULL), (dict(vn=None), NULL), (dict(out=None), NULL), (dict(ts=100), SHAPE),
    (dict(ts=4 * 128 + 4), ALIGN), (dict(kn=MIS), ALIGN), (dict(d=96), UNSUP), (dict(B=0), OK),
    (dict(B=0, kn=None), OK),
])
def test_decode_step_argument_checks(fp8, kw, code):
    if fp8:
        kw = dict(kw)
        if "block_stride" not in kw:
            kw["block_stride"] = 16 * 4 * 128
    assert _step(fp8, **kw) == code


def test_decode_step_fp8_specific_checks():
    assert _step(True, dtype=0) == DTYPE
    assert _step(True, ks=None) == NULL
    assert _step(False, dtype=7) == DTYPE


def test_graph_handle_checks():
    lib = P.lib()
    assert lib.pa_graph_begin(None, None) == NULL
    assert lib.pa_graph_end(None) == NULL
    assert lib.pa_graph_launch(None, None) == NULL
    lib.pa_graph_destroy(None)                       # no-op


def test_binding_raises_on_error_status():
    err = P.PagedAttentionError("pa_decode", 4)
    assert "PA_ERR_UNSUPPORTED" in str(err) and err.status == 4


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libpagedattn.so")
    with pytest.raises(P.LibraryNotBuilt):
        B.lib()
