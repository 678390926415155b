"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects invalid arguments with the documented status before touching the
device.  No valid call is ever made here (there is no GPU): every call below
fails validation, so the fake pointer values are never dereferenced."""

import ctypes
import os
import re

import pytest

import sliding_window_attention_swa_amd as swa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("swa.h", "swa_calib.h")]

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
P = 0x10000  # aligned, never dereferenced
MIS = P + 8  # misaligned


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(swa.LIB_PATH):
        from sliding_window_attention_swa_amd import build
        build.build(verbose=False)
    return swa.load()


def declared_functions(headers=None):
    names = set()
    for path in headers or HEADERS:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(swa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_headers_declare_the_entry_points():
    assert declared_functions(HEADERS[:1]) == sorted([
        "swa_prefill", "swa_cache_append", "swa_decode", "swa_decode_workspace_bytes",
        "swa_status_string", "swa_cache_append_chunk", "swa_prefill_chunk",
        "swa_prefill_dilated", "swa_prefill_global", "swa_prefill_global_workspace_bytes",
        "swa_prefill_dilated_global",
        "swa_decode_sinks", "swa_decode_sinks_workspace_bytes", "swa_decode_noalloc"])
    # the calibration kernels compute nothing of the method: a header of their own
    assert declared_functions(HEADERS[1:]) == ["swa_calib_mfma_bf16", "swa_calib_stream_read",
                                               "swa_calib_vector"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def prefill(lib, q=P, k=P, v=P, out=P, T=16, W=4, Hq=4, Hkv=2, d=64, mode=0, scale=0.125,
            dtype=1):
    return lib.swa_prefill(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(out=None), INVALID), (dict(q=MIS), INVALID), (dict(out=MIS), INVALID),
    (dict(T=0), INVALID), (dict(T=-3), INVALID), (dict(W=0), INVALID), (dict(Hq=0), INVALID),
    (dict(Hkv=0), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(mode=2), UNSUPPORTED),
    (dict(dtype=2), UNSUPPORTED), (dict(dtype=-1), UNSUPPORTED),
    (dict(T=2**30, Hq=2**10, Hkv=1), UNSUPPORTED),
    # sequences past 2^29 rows (the int32 index range of a block's key span)
    (dict(T=2**29 + 1, Hq=1, Hkv=1), UNSUPPORTED), (dict(T=2**31 - 1, Hq=1, Hkv=1), UNSUPPORTED),
    # |scale| past 1024 (the fp32 exponent s * c - m * c keeps its precision)
    (dict(scale=1024.5), INVALID), (dict(scale=-2000.0), INVALID), (dict(scale=1e9), INVALID),
    (dict(scale=-3e38), INVALID),
])
def test_prefill_rejects(lib, kw, status):
    assert prefill(lib, **kw) == status


def prefill_dilated(lib, q=P, k=P, v=P, out=P, T=16, W=4, Hq=4, Hkv=2, d=64, mode=0, scale=0.125,
                    dil=2, dtype=1):
    return lib.swa_prefill_dilated(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dil, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(out=None), INVALID), (dict(k=MIS), INVALID),
    (dict(T=0), INVALID), (dict(W=0), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(dil=0), INVALID), (dict(dil=-2), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(mode=2), UNSUPPORTED), (dict(dtype=9), UNSUPPORTED),
    (dict(dil=2**17, d=128), UNSUPPORTED),  # 64 strided rows beyond 32-bit byte offsets
    (dict(T=2**30, Hq=2**10, Hkv=1, dil=1), UNSUPPORTED),
])
def test_prefill_dilated_rejects(lib, kw, status):
    assert prefill_dilated(lib, **kw) == status


def prefill_global(lib, q=P, k=P, v=P, out=P, T=16, W=4, Hq=4, Hkv=2, d=64, mode=0, scale=0.125,
                   gpos=P, G=2, ws=P, ws_bytes=None, dtype=1):
    if ws_bytes is None:
        ws_bytes = lib.swa_prefill_global_workspace_bytes(T, Hq, G, d) if G > 0 and Hq > 0 and T > 0 else 0
    return lib.swa_prefill_global(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, gpos, G, ws,
                                  ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(gpos=None), INVALID), (dict(gpos=MIS), INVALID),
    (dict(G=-1), INVALID), (dict(T=0), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(d=40), UNSUPPORTED), (dict(mode=3), UNSUPPORTED),
    (dict(dtype=4), UNSUPPORTED), (dict(ws=None), WORKSPACE), (dict(ws=MIS), WORKSPACE),
    (dict(ws_bytes=16), WORKSPACE),
    (dict(T=2**24, d=128), UNSUPPORTED),  # gathered rows beyond 32-bit byte offsets
])
def test_prefill_global_rejects(lib, kw, status):
    assert prefill_global(lib, **kw) == status


def test_global_workspace_bytes(lib):
    f = lib.swa_prefill_global_workspace_bytes
    assert f(0, 8, 2, 64) == 0 and f(100, 0, 2, 64) == 0 and f(100, 8, 0, 64) == 0
    assert f(100, 8, 2, 48) == 0
    for T, Hq, G, d in [(4096, 48, 8, 64), (16, 1, 1, 32), (100000, 32, 3, 128)]:
        n = f(T, Hq, G, d)
        assert n > 0 and n % (4 * (d + 2) * G * Hq) == 0
        assert 1 <= n // (4 * (d + 2) * G * Hq) <= max(1, (T + 63) // 64)


def dilated_global(lib, q=P, k=P, v=P, out=P, T=64, W=8, Hq=4, Hkv=2, d=64, mode=1, scale=0.125,
                   dil=2, gpos=P, G=3, ws=P, ws_bytes=1 << 30, dtype=1):
    return lib.swa_prefill_dilated_global(q, k, v, out, T, W, Hq, Hkv, d, mode, scale, dil, gpos,
                                          G, ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(gpos=None), INVALID), (dict(gpos=MIS), INVALID),
    (dict(G=-1), INVALID), (dict(T=0), INVALID), (dict(Hq=6, Hkv=4), INVALID),
    (dict(dil=0), INVALID), (dict(dil=-2), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(d=40), UNSUPPORTED), (dict(mode=2), UNSUPPORTED), (dict(dtype=3), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws=MIS), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
    (dict(dil=2**20, d=128), UNSUPPORTED),  # a tile's rows beyond 32-bit byte offsets
    (dict(T=2**24, d=128), UNSUPPORTED),
    # G = 0 is swa_prefill_dilated (its checks), dilation 1 is swa_prefill_global
    (dict(G=0, gpos=None, ws=None, ws_bytes=0, dil=0), INVALID),
    (dict(G=0, gpos=None, ws=None, ws_bytes=0, d=48), UNSUPPORTED),
    (dict(dil=1, ws=None), WORKSPACE), (dict(dil=1, mode=5), UNSUPPORTED),
])
def test_prefill_dilated_global_rejects(lib, kw, status):
    assert dilated_global(lib, **kw) == status


def test_prefill_global_without_globals_is_prefill_validation(lib):
    # G = 0 takes swa_prefill's path (and its checks): no positions or workspace needed
    assert prefill_global(lib, G=0, gpos=None, ws=None, ws_bytes=0, T=0) == INVALID
    assert prefill_global(lib, G=0, gpos=None, ws=None, ws_bytes=0, d=48) == UNSUPPORTED


def append(lib, kr=P, vr=P, pos=P, kn=P, vn=P, B=2, Hkv=2, W=8, d=64, dtype=1):
    return lib.swa_cache_append(kr, vr, pos, kn, vn, B, Hkv, W, d, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kr=None), INVALID), (dict(vr=None), INVALID), (dict(pos=None), INVALID),
    (dict(kn=None), INVALID), (dict(vn=None), INVALID), (dict(kr=MIS), INVALID),
    (dict(pos=MIS), INVALID), (dict(B=0), INVALID), (dict(Hkv=0), INVALID), (dict(W=0), INVALID),
    (dict(d=16), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED),
])
def test_append_rejects(lib, kw, status):
    assert append(lib, **kw) == status


def append_chunk(lib, kr=P, vr=P, pos=P, k=P, v=P, B=2, n=5, Hkv=2, W=8, d=64, dtype=1):
    return lib.swa_cache_append_chunk(kr, vr, pos, k, v, B, n, Hkv, W, d, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(kr=None), INVALID), (dict(vr=None), INVALID), (dict(pos=None), INVALID),
    (dict(k=None), INVALID), (dict(v=None), INVALID), (dict(vr=MIS), INVALID),
    (dict(k=MIS), INVALID), (dict(B=0), INVALID), (dict(n=0), INVALID), (dict(n=-1), INVALID),
    (dict(Hkv=0), INVALID), (dict(W=0), INVALID), (dict(d=8), UNSUPPORTED),
    (dict(dtype=2), UNSUPPORTED),
    (dict(B=65536, Hkv=1024), UNSUPPORTED),  # 2^31 or more 16-byte chunks to write
])
def test_append_chunk_rejects(lib, kw, status):
    assert append_chunk(lib, **kw) == status


def prefill_chunk(lib, q=P, k=P, v=P, kr=P, vr=P, pos=P, out=P, B=2, n=16, W=8, Hq=4, Hkv=2,
                  d=64, scale=0.125, dtype=1):
    return lib.swa_prefill_chunk(q, k, v, kr, vr, pos, out, B, n, W, Hq, Hkv, d, scale, dtype,
                                 None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(kr=None), INVALID), (dict(vr=None), INVALID), (dict(pos=None), INVALID),
    (dict(out=None), INVALID), (dict(q=MIS), INVALID), (dict(kr=MIS), INVALID),
    (dict(pos=MIS), INVALID), (dict(out=MIS), INVALID), (dict(B=0), INVALID),
    (dict(n=0), INVALID), (dict(W=-2), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(d=16), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED),
    (dict(W=2**24, d=128), UNSUPPORTED),  # ring rows beyond 32-bit byte offsets
    (dict(B=2**16, n=2**20, Hq=2**10, Hkv=1), UNSUPPORTED),
])
def test_prefill_chunk_rejects(lib, kw, status):
    assert prefill_chunk(lib, **kw) == status


def decode(lib, q=P, kr=P, vr=P, pos=P, out=P, B=2, Hq=8, Hkv=2, W=4096, d=64, scale=0.125,
           dtype=1, ws=P, ws_bytes=None):
    # the default sizes split the ring, so a workspace is required
    if ws_bytes is None:
        ws_bytes = lib.swa_decode_workspace_bytes(B, Hq, W, d) if B > 0 and Hq > 0 and W > 0 else 0
    return lib.swa_decode(q, kr, vr, pos, out, B, Hq, Hkv, W, d, scale, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kr=None), INVALID), (dict(vr=None), INVALID),
    (dict(pos=None), INVALID), (dict(out=None), INVALID), (dict(vr=MIS), INVALID),
    (dict(B=0), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=0), INVALID), (dict(W=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(d=96), UNSUPPORTED), (dict(dtype=3), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws=MIS), WORKSPACE), (dict(ws_bytes=0), WORKSPACE),
])
def test_decode_rejects(lib, kw, status):
    assert decode(lib, **kw) == status


def decode_noalloc(lib, q=P, kr=P, vr=P, pos=P, out=P, B=2, Hq=8, Hkv=2, W=4096, d=64,
                   scale=0.125, dtype=1):
    return lib.swa_decode_noalloc(q, kr, vr, pos, out, B, Hq, Hkv, W, d, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(kr=None), INVALID), (dict(vr=None), INVALID),
    (dict(pos=None), INVALID), (dict(out=None), INVALID), (dict(q=MIS), INVALID),
    (dict(out=MIS), INVALID), (dict(B=0), INVALID), (dict(Hq=0), INVALID), (dict(Hkv=-1), INVALID),
    (dict(W=0), INVALID), (dict(Hq=6, Hkv=4), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(scale=1025.0), INVALID), (dict(d=16), UNSUPPORTED), (dict(dtype=5), UNSUPPORTED),
])
def test_decode_noalloc_rejects(lib, kw, status):
    assert decode_noalloc(lib, **kw) == status


def test_decode_noalloc_scratch_holds_every_split_decode(lib):
    """The per-GPU scratch (4 MiB) holds the partials of any decode that
    splits its ring: at most 4096 records of d + 2 floats."""
    worst = 0
    for B in (1, 2, 3, 5, 7, 16, 31, 64, 100, 511, 1023, 2047):
        for Hq in (1, 2, 3, 4, 8):
            for W in (65, 1000, 4096, 1 << 20):
                worst = max(worst, lib.swa_decode_workspace_bytes(B, Hq, W, 128))
    assert 0 < worst <= 4096 * 130 * 4 <= 4 << 20


def decode_sinks(lib, q=P, kr=P, vr=P, ks=P, vs=P, S=4, pos=P, out=P, B=2, Hq=8, Hkv=2, W=64,
                 d=64, scale=0.125, dtype=1, ws=P, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.swa_decode_sinks_workspace_bytes(B, Hq, W, d) if B > 0 and Hq > 0 and W > 0 else 0
    return lib.swa_decode_sinks(q, kr, vr, ks, vs, S, pos, out, B, Hq, Hkv, W, d, scale, dtype, ws,
                                ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), INVALID), (dict(vs=None), INVALID), (dict(ks=MIS), INVALID),
    (dict(S=-1), INVALID), (dict(q=None), INVALID), (dict(B=0), INVALID),
    (dict(Hq=6, Hkv=4), INVALID), (dict(d=16), UNSUPPORTED), (dict(dtype=8), UNSUPPORTED),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=64), WORKSPACE),
])
def test_decode_sinks_rejects(lib, kw, status):
    assert decode_sinks(lib, **kw) == status


def test_decode_sinks_workspace_is_one_split_more_than_decode(lib):
    for B, Hq, W, d in [(64, 32, 4096, 128), (1, 2, 100, 64), (3, 8, 37, 32)]:
        per_split = 4 * (d + 2) * B * Hq
        # the plain decode keeps no partial record when it has one split
        splits = max(1, lib.swa_decode_workspace_bytes(B, Hq, W, d) // per_split)
        assert lib.swa_decode_sinks_workspace_bytes(B, Hq, W, d) == (splits + 1) * per_split


def test_decode_rejects_one_byte_short_workspace(lib):
    need = lib.swa_decode_workspace_bytes(2, 8, 4096, 64)
    assert need > 0
    assert decode(lib, ws_bytes=need - 1) == WORKSPACE


def test_workspace_bytes(lib):
    f = lib.swa_decode_workspace_bytes
    assert f(0, 8, 64, 64) == 0 and f(2, 0, 64, 64) == 0 and f(2, 8, 0, 64) == 0
    assert f(2, 8, 64, 48) == 0
    # one split (enough heads to fill the GPU, or a ring of at most 64 slots):
    # the kernel writes the output itself and needs no workspace (the
    # Mistral-7B decode: 64 sequences x 32 heads)
    assert f(64, 32, 4096, 128) == 0 and f(1, 1, 4, 64) == 0 and f(16, 128, 4096, 64) == 0
    for B, Hq, W, d in [(1, 32, 4096, 128), (3, 5, 100, 32), (2, 8, 4096, 64)]:
        n = f(B, Hq, W, d)
        # whole fp32 partial records (d accumulators + max + sum) per split
        assert n > 0 and n % (4 * (d + 2) * B * Hq) == 0
        splits = n // (4 * (d + 2) * B * Hq)
        assert 2 <= splits <= (W + 63) // 64


def test_decode_without_workspace_only_when_none_is_needed(lib):
    # a call that needs partials rejects a missing workspace ...
    assert lib.swa_decode_workspace_bytes(2, 8, 4096, 64) > 0
    assert decode(lib, ws=None, ws_bytes=0) == WORKSPACE
    # ... and one that needs none gets past the workspace check (it then fails
    # on the head count, so nothing is launched)
    assert lib.swa_decode_workspace_bytes(64, 32, 4096, 128) == 0
    assert decode(lib, B=64, Hq=33, Hkv=8, W=4096, d=128, ws=None, ws_bytes=0) == INVALID


def calib_mfma(lib, ops=P, nbytes=65536, sink=P, n_wg=8, iters=10):
    return lib.swa_calib_mfma_bf16(ops, nbytes, sink, n_wg, iters, None)


@pytest.mark.parametrize("kw,status", [
    (dict(ops=None), INVALID), (dict(sink=None), INVALID), (dict(ops=MIS), INVALID),
    (dict(sink=MIS), INVALID), (dict(nbytes=0), INVALID), (dict(nbytes=8), INVALID),
    (dict(nbytes=65540), INVALID), (dict(n_wg=0), INVALID), (dict(n_wg=2**20 + 1), INVALID),
    (dict(iters=-1), INVALID), (dict(nbytes=2**36), UNSUPPORTED),
])
def test_calib_mfma_rejects(lib, kw, status):
    assert calib_mfma(lib, **kw) == status


def calib_read(lib, src=P, nbytes=2**20, sink=P, n_wg=8):
    return lib.swa_calib_stream_read(src, nbytes, sink, n_wg, None)


@pytest.mark.parametrize("kw,status", [
    (dict(src=None), INVALID), (dict(sink=None), INVALID), (dict(src=MIS), INVALID),
    (dict(sink=MIS), INVALID), (dict(nbytes=0), INVALID), (dict(nbytes=2**20 + 4), INVALID),
    (dict(n_wg=0), INVALID), (dict(n_wg=2**24), UNSUPPORTED),
])
def test_calib_read_rejects(lib, kw, status):
    assert calib_read(lib, **kw) == status


def calib_vector(lib, op=0, sink=P, n_wg=8, iters=10):
    return lib.swa_calib_vector(op, sink, n_wg, iters, None)


@pytest.mark.parametrize("kw,status", [
    (dict(op=-1), INVALID), (dict(op=2), INVALID), (dict(sink=None), INVALID),
    (dict(sink=MIS), INVALID), (dict(n_wg=0), INVALID), (dict(n_wg=2**20 + 1), INVALID),
    (dict(iters=-1), INVALID), (dict(op=1, iters=-5), INVALID),
])
def test_calib_vector_rejects(lib, kw, status):
    assert calib_vector(lib, **kw) == status


def test_status_strings(lib):
    assert swa.status_string(0) == "ok"
    texts = {swa.status_string(s) for s in (0, -1, -2, -3, -4)}
    assert len(texts) == 5
    assert swa.status_string(-99) == "unknown status"


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(swa, "_lib", None)
    monkeypatch.setattr(swa, "LIB_PATH", "/nonexistent/libswa.so")
    with pytest.raises(RuntimeError, match="libswa.so not found"):
        swa.load()
